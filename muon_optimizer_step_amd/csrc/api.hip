// Host side of the Muon step library: argument validation, shape grouping,
// workspace layout and the launch sequence behind the C ABI in muonstep.h.
//
// One muon_step enqueues, per lane (the caller's stream and, when the shape
// groups split over two, an internal stream forked from it and joined back):
//   prep  (per-row momentum, MuonEq-R row norm, NS input X0 short side first)
//   frob  (per-matrix Frobenius scale from the per-row sums; folded into the
//   first ns_gram unless a launch holds more than kMaxFrobSlots matrices)
//   for each NS iteration: ns_gram, ns_square, ns_update (the lane's shape
//   groups batched in one launch per phase)
//   apply (decoupled weight decay + shape-scaled update, and the EMA; inside
//   the last ns_update unless a launch holds more than kMaxFused matrices)
// ema_update, ema_swap and adamw_step enqueue one multi-tensor launch per
// table chunk on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/muonstep.h"
#include "common.h"
#include "kernels.h"

namespace muon {
namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------- profiling
struct PendingEvent {
    std::string name;
    hipEvent_t start, stop;
};
struct ProfileTotal {
    int64_t count = 0;
    double ms = 0.0;
};
std::mutex g_prof_mu;
bool g_prof_enabled = false;
std::vector<PendingEvent> g_pending;
std::vector<hipEvent_t> g_event_pool;
std::vector<std::pair<std::string, ProfileTotal>> g_totals;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Runs `launch` (which returns the launch's hipError_t) bracketed by events
// when profiling is on.
template <typename F>
hipError_t timed_launch(const char* name, hipStream_t s, F launch) {
    bool prof;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        prof = g_prof_enabled;
    }
    if (!prof) return launch();
    hipEvent_t e0, e1;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        e0 = take_event();
        e1 = take_event();
    }
    if (!e0 || !e1) return hipErrorOutOfMemory;
    hipError_t err = hipEventRecord(e0, s);
    if (err != hipSuccess) return err;
    err = launch();
    if (err != hipSuccess) return err;
    err = hipEventRecord(e1, s);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_pending.push_back({name, e0, e1});
    return hipSuccess;
}

// ------------------------------------------------------------- NS lanes
// The matrices are independent NS problems.  Their shape groups are spread
// over up to kLanes streams (the caller's stream and internal non-blocking streams of
// default priority), forked from and joined back into the caller's stream with
// events, so that short chains (small matrices) fill the compute units the
// long ones leave idle.  Nothing waits on the host.
#ifndef NS_LANES
#define NS_LANES 2
#endif
constexpr int kLanes = NS_LANES;
struct LaneSet {
    hipStream_t stream[kLanes] = {};   // [0] unused: lane 0 is the caller's stream
    hipEvent_t fork = nullptr;
    hipEvent_t join[kLanes] = {};
    bool ready = false;
};
std::mutex g_lane_mu;
std::map<int, LaneSet> g_lanes;

hipError_t lanes_for_device(int dev, LaneSet*& out) {
    LaneSet& L = g_lanes[dev];
    if (!L.ready) {
        hipError_t e = hipSuccess;
        for (int i = 1; i < kLanes && e == hipSuccess; ++i) {
            e = hipStreamCreateWithFlags(&L.stream[i], hipStreamNonBlocking);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&L.join[i], hipEventDisableTiming);
        }
        if (e == hipSuccess) e = hipEventCreateWithFlags(&L.fork, hipEventDisableTiming);
        if (e != hipSuccess) {
            // release what was created; the next call starts over
            for (int i = 1; i < kLanes; ++i) {
                if (L.stream[i]) (void)hipStreamDestroy(L.stream[i]);
                if (L.join[i]) (void)hipEventDestroy(L.join[i]);
            }
            if (L.fork) (void)hipEventDestroy(L.fork);
            L = LaneSet();
            return e;
        }
        L.ready = true;
    }
    out = &L;
    return hipSuccess;
}

// ------------------------------------------------------------- planning
struct Group {
    int m, n;        // short side, long side
    int M, N;        // padded
    int count = 0;
    size_t x_off[2], xl_off[2], ah_off, al_off, b_off, bl_off;
    bool comp = false;    // run the compensated bf16 products
    int scale_begin = 0;  // index of slot 0 in the scale array
};

struct Plan {
    std::vector<Group> groups;
    std::vector<std::vector<int>> members;  // tensors of each group, by slot
    std::vector<int> group_of, slot_of;
    std::vector<size_t> rowsq_off;  // in floats
    size_t rowsq_base = 0;          // byte offset of the rowsq array
    size_t scale_base = 0;          // byte offset of the per-matrix scale array
    // persistent chain over the base-precision bf16 groups (chain.hip)
    std::vector<std::vector<int>> chain_launch_groups;  // groups of each chain launch (<= kMaxGroups)
    int chain_mats = 0;             // matrices in those groups
    size_t chain_rec_base = 0;      // byte offset of the ChainMat records
    size_t chain_ctr_base = 0;      // byte offset of the counters (+ one status block per launch)
    int chain_ctr_words = 0;
    size_t bytes = 0;
};

int transposed_rb(int cols) {
    // stored rows per workgroup when X0 is the transpose: rb * (cols + 1) floats
    // of LDS (at most 64 KiB; more costs occupancy), so that each X0 row
    // segment a workgroup writes is rb * 2 bytes per bf16 plane
    int rb = 64;
    while (rb > 1 && (size_t)rb * (cols + 1) * sizeof(float) > kTransposeLdsBytes) rb >>= 1;
    return rb;
}

// mode: the ns_precision argument.  Storage is bf16 hi/lo planes except in fp32 mode.
void make_plan(const muon_tensor_t* t, int n, int mode, Plan& p) {
    const int precision = mode == kModeFp32 ? kNsFp32 : kNsBf16;
    std::map<std::pair<int, int>, int> index;
    p.group_of.resize(n);
    p.slot_of.resize(n);
    p.rowsq_off.resize(n);
    size_t rowsq_total = 0;
    for (int i = 0; i < n; ++i) {
        const int m = std::min(t[i].rows, t[i].cols), nn = std::max(t[i].rows, t[i].cols);
        auto key = std::make_pair(m, nn);
        auto it = index.find(key);
        int g;
        if (it == index.end()) {
            g = (int)p.groups.size();
            index[key] = g;
            Group G;
            G.m = m;
            G.n = nn;
            G.M = pad_to_tile(m);
            G.N = pad_to_tile(nn);
            G.comp = mode == kModeBf16x3 || (mode == kModeBf16 && m < kCompensateBelow);
            p.groups.push_back(G);
        } else {
            g = it->second;
        }
        p.group_of[i] = g;
        p.slot_of[i] = p.groups[g].count++;
        if ((int)p.members.size() <= g) p.members.resize(g + 1);
        p.members[g].push_back(i);
        p.rowsq_off[i] = rowsq_total;
        rowsq_total += (size_t)t[i].rows;
    }
    const size_t xe = precision == kNsBf16 ? 2 : 4;  // bytes per element of an X / A / B plane
    size_t off = 0;
    for (Group& G : p.groups) {
        const size_t xplane = align256((size_t)G.count * G.M * G.N * xe);
        const size_t aplane = align256((size_t)G.count * G.M * G.M * xe);
        for (int k = 0; k < 2; ++k) { G.x_off[k] = off; off += xplane; }
        if (precision == kNsBf16) {
            for (int k = 0; k < 2; ++k) { G.xl_off[k] = off; off += xplane; }
        } else {
            G.xl_off[0] = G.x_off[0];
            G.xl_off[1] = G.x_off[1];
        }
        G.ah_off = off; off += aplane;
        if (precision == kNsBf16) { G.al_off = off; off += aplane; } else { G.al_off = G.ah_off; }
        G.b_off = off; off += aplane;
        if (precision == kNsBf16) { G.bl_off = off; off += aplane; } else { G.bl_off = G.b_off; }
    }
    int scale_count = 0;
    for (Group& G : p.groups) { G.scale_begin = scale_count; scale_count += G.count; }
    p.scale_base = off;
    off += align256((size_t)scale_count * sizeof(float));
    p.rowsq_base = off;
    off += align256(rowsq_total * sizeof(float));
    // chain launches: the base bf16 groups, kMaxGroups per launch
    if (precision == kNsBf16) {
        for (int g = 0; g < (int)p.groups.size(); ++g) {
            if (p.groups[g].comp) continue;
            if (p.chain_launch_groups.empty() || (int)p.chain_launch_groups.back().size() == kMaxGroups)
                p.chain_launch_groups.emplace_back();
            p.chain_launch_groups.back().push_back(g);
            p.chain_mats += p.groups[g].count;
        }
    }
    p.chain_rec_base = off;
    off += align256((size_t)p.chain_mats * sizeof(ChainMat));
    p.chain_ctr_base = off;
    p.chain_ctr_words = (p.chain_mats + (int)p.chain_launch_groups.size()) * kChainCtrWords;
    off += align256((size_t)p.chain_ctr_words * sizeof(uint32_t));
    p.bytes = off;
}

// ------------------------------------------------------------- validation
struct Span {
    uintptr_t lo, hi;
    int tensor;
};

int check_overlaps(std::vector<Span>& spans, const char* what) {
    std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < spans.size(); ++i) {
        if (spans[i].lo < spans[i - 1].hi)
            return fail(MUON_ERR_UNSUPPORTED, "%s: buffers of tensors %d and %d overlap", what,
                        spans[i - 1].tensor, spans[i].tensor);
    }
    return MUON_OK;
}

int validate_tensors(const muon_tensor_t* t, int32_t n, int32_t precision) {
    if (!t) return fail(MUON_ERR_INVALID_ARG, "tensors is NULL");
    if (n <= 0 || n > MUON_MAX_TENSORS) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, MUON_MAX_TENSORS);
    if (precision != MUON_NS_BF16 && precision != MUON_NS_FP32 && precision != MUON_NS_BF16X3)
        return fail(MUON_ERR_INVALID_ARG, "ns_precision = %d is not MUON_NS_BF16, MUON_NS_FP32 or MUON_NS_BF16X3", precision);
    for (int i = 0; i < n; ++i) {
        const muon_tensor_t& x = t[i];
        if (x.rows <= 0 || x.cols <= 0)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: rows = %d, cols = %d must be positive", i, x.rows, x.cols);
        if (std::min(x.rows, x.cols) > MUON_MAX_SHORT_SIDE || std::max(x.rows, x.cols) > MUON_MAX_LONG_SIDE)
            return fail(MUON_ERR_UNSUPPORTED, "tensor %d: shape %d x %d beyond the limits (short side <= %d, long side <= %d)",
                        i, x.rows, x.cols, MUON_MAX_SHORT_SIDE, MUON_MAX_LONG_SIDE);
    }
    return MUON_OK;
}

int validate_pointers(const muon_tensor_t* t, int32_t n) {
    std::vector<Span> spans;
    spans.reserve(5 * (size_t)n);
    for (int i = 0; i < n; ++i) {
        const muon_tensor_t& x = t[i];
        if (!x.param || !x.grad || !x.momentum)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: param, grad and momentum must be non-NULL", i);
        const size_t bytes = (size_t)x.rows * x.cols * sizeof(float);
        const void* ptrs[5] = {x.param, x.grad, x.momentum, x.update_out, x.ema};
        for (int k = 0; k < 5; ++k) {
            if (!ptrs[k]) continue;
            if (reinterpret_cast<uintptr_t>(ptrs[k]) % sizeof(float))
                return fail(MUON_ERR_INVALID_ARG, "tensor %d: pointer %d is not 4-byte aligned", i, k);
            const uintptr_t lo = reinterpret_cast<uintptr_t>(ptrs[k]);
            spans.push_back({lo, lo + bytes, i});
        }
    }
    return check_overlaps(spans, "muon_step");
}

// Scale exponents of the base bf16 square's e4m3 operands, per NS iteration.
// X0 has sigma_max <= 1 (Frobenius scaling); iteration k maps every singular
// value through p_k(s) = a s + b s^3 + c s^5, so sigma_max(X_k) is bounded by
// the maximum of |p| over [0, bound of X_{k-1}] (sampled, with a margin for
// the bf16 rounding), and |A_ij| <= sigma_max(X_k)^2.  A hi is scaled by 2^sa
// and A lo (at most 2^-8 |A|) by 2^(sa + 8) so that both stay under 224 in
// e4m3 (which saturates at 448).
void f8_scale_exponents(const float* coeffs, int ns_steps, int* sa) {
    double bound = 1.0;   // sigma_max of X_k
    for (int k = 0; k < ns_steps; ++k) {
        if (!(bound <= 1e30)) bound = 1e30;   // also catches NaN: far past any useful table
        const double amax = bound * bound * 1.05;
        double e = 64.0;   // clamped before the conversion to int
        if (amax > 0.0) e = std::max(-64.0, std::min(64.0, std::floor(std::log2(224.0) - std::log2(amax))));
        sa[k] = (int)e;
        const double a = coeffs[3 * k], b = coeffs[3 * k + 1], c = coeffs[3 * k + 2];
        const double hi = bound * 1.02;
        double m = 0.0;
        for (int i = 0; i <= 4096; ++i) {
            const double x = hi * i / 4096.0, x2 = x * x;
            m = std::max(m, std::fabs(x * (a + x2 * (b + c * x2))));
        }
        bound = m * 1.02;
    }
}

// Streaming tensors (EMA, AdamW): at most 2^30 workgroups per launch, so a
// single tensor may hold at most this many elements (4 Ti elements; far above
// any device memory).
constexpr int64_t kMaxStreamElems = ((int64_t)1 << 30) * 1024;

// ------------------------------------------------------------- schedules
// Everything muon_step derives from the tensor list alone (validation of the
// pointers, shape groups, workspace layout, lanes, launch sets, the chain's
// XCD binding and matrix records) is a Schedule, cached by the call's
// signature: the tensor descriptors, the precision and the workspace.  A call
// whose signature matches a cached one only checks its scalars and enqueues.
struct Part {
    int group, s0, s1;  // slots [s0, s1) of the group
    int lane;
};
struct NsLaunchSet {
    int lane, comp;
    std::vector<int> parts;
};
struct ChainLaunch {
    ChainArgs a;          // groups, records, counters, XCD table; scalars set per call
};
struct Schedule {
    std::vector<uint64_t> key;
    Plan p;
    int mode = 0, prec = 0;
    // per-phase path (lanes), for the groups the chain does not take
    std::vector<Part> parts;
    int nlanes = 1;
    std::vector<NsLaunchSet> sets;
    std::vector<std::vector<int>> mine;        // tensors of each lane (prep)
    std::vector<std::vector<int>> legacy;      // tensors of each lane outside the chain
    int max_set_count = 0;                     // matrices of the largest launch set
    // chain
    bool chain = false;
    std::vector<ChainLaunch> chains;
    std::vector<ChainSetupArgs> setups;
    // e4m3 scale exponents of the last coefficient table seen
    std::vector<float> f8_coeffs;
    int f8_sa[MUON_MAX_NS_STEPS] = {};
};

std::mutex g_sched_mu;
std::vector<std::shared_ptr<Schedule>> g_sched;   // most recently used last
constexpr size_t kMaxSchedules = 8;
int64_t g_sched_built = 0, g_sched_hits = 0;

std::vector<uint64_t> schedule_key(const muon_tensor_t* t, int n, int mode, int schedule, const void* ws,
                                   size_t ws_bytes) {
    std::vector<uint64_t> k;
    k.reserve(5 + 6 * (size_t)n);
    k.push_back((uint64_t)n);
    k.push_back((uint64_t)mode);
    k.push_back((uint64_t)schedule);
    k.push_back(reinterpret_cast<uintptr_t>(ws));
    k.push_back((uint64_t)ws_bytes);
    for (int i = 0; i < n; ++i) {
        k.push_back(reinterpret_cast<uintptr_t>(t[i].param));
        k.push_back(reinterpret_cast<uintptr_t>(t[i].grad));
        k.push_back(reinterpret_cast<uintptr_t>(t[i].momentum));
        k.push_back(reinterpret_cast<uintptr_t>(t[i].update_out));
        k.push_back(reinterpret_cast<uintptr_t>(t[i].ema));
        k.push_back(((uint64_t)(uint32_t)t[i].rows << 32) | (uint32_t)t[i].cols);
    }
    return k;
}

// How the Newton-Schulz iterations of the base bf16 groups are scheduled:
// MUON_NS_SCHEDULE_PHASES (one launch per phase, the default) or
// MUON_NS_SCHEDULE_CHAIN (the persistent chain).  MUON_CHAIN=1 in the
// environment selects the chain at load time; muon_set_ns_schedule changes it.
std::atomic<int> g_ns_schedule{[] {
    const char* v = std::getenv("MUON_CHAIN");
    return (v && v[0] == '1') ? MUON_NS_SCHEDULE_CHAIN : MUON_NS_SCHEDULE_PHASES;
}()};
bool chain_allowed(int schedule) { return schedule == MUON_NS_SCHEDULE_CHAIN; }

// Compute units of device dev (cached); 0 if unknown.
int device_cus(int dev) {
    static std::mutex mu;
    static std::map<int, int> cache;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    cache[dev] = cus;
    return cus;
}

double ns_flops_per_iter(const Group& G) {
    return 4.0 * G.M * (double)G.M * G.N + 2.0 * G.M * (double)G.M * G.M;
}

// The chain binds a matrix to one XCD (an eighth of the GPU).  It is not used
// when one matrix alone holds more than half of the NS work of a call and is
// large enough for the whole GPU to matter (a single very large matrix runs
// faster on the per-phase kernels, which spread its tiles over every XCD).
bool chain_worthwhile(const Plan& p) {
    double total = 0.0, biggest = 0.0;
    for (const auto& lg : p.chain_launch_groups)
        for (int g : lg) {
            total += ns_flops_per_iter(p.groups[g]) * p.groups[g].count;
            biggest = std::max(biggest, ns_flops_per_iter(p.groups[g]));
        }
    if (total <= 0.0) return false;
    return biggest <= 0.5 * total || biggest < 4e9;
}

float shape_scale_of(const muon_tensor_t& x) {
    return (float)std::sqrt(std::max(1.0, (double)x.rows / (double)x.cols));
}
bool vec_ok(const muon_tensor_t& x) {
    // 16-byte accesses to the caller's W / O / EMA rows
    return (x.cols % 4 == 0) && (reinterpret_cast<uintptr_t>(x.param) % 16 == 0) &&
           (reinterpret_cast<uintptr_t>(x.update_out) % 16 == 0) && (reinterpret_cast<uintptr_t>(x.ema) % 16 == 0);
}

// Validation of the tensor list and the workspace, then every derived table.
int build_schedule(const muon_tensor_t* tensors, int n, int mode, int schedule, void* workspace,
                   size_t workspace_bytes, Schedule& S) {
    int rc = validate_pointers(tensors, n);
    if (rc) return rc;
    Plan& p = S.p;
    make_plan(tensors, n, mode, p);
    if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL (needs %zu bytes)", p.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(MUON_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < p.bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, p.bytes);
    {
        // the workspace must not overlap any tensor
        const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace), whi = wlo + p.bytes;
        for (int i = 0; i < n; ++i) {
            const muon_tensor_t& x = tensors[i];
            const size_t bytes = (size_t)x.rows * x.cols * sizeof(float);
            const void* ptrs[5] = {x.param, x.grad, x.momentum, x.update_out, x.ema};
            for (int k = 0; k < 5; ++k) {
                if (!ptrs[k]) continue;
                const uintptr_t lo = reinterpret_cast<uintptr_t>(ptrs[k]);
                if (lo < whi && wlo < lo + bytes)
                    return fail(MUON_ERR_UNSUPPORTED, "tensor %d overlaps the workspace", i);
            }
        }
    }
    S.mode = mode;
    S.prec = mode == MUON_NS_FP32 ? kNsFp32 : kNsBf16;
    S.chain = chain_allowed(schedule) && !p.chain_launch_groups.empty() && chain_worthwhile(p);
    const int ngroups = (int)p.groups.size();
    std::vector<char> in_chain(ngroups, 0);
    if (S.chain)
        for (const auto& lg : p.chain_launch_groups)
            for (int g : lg) in_chain[g] = 1;

    // ---- lanes of the per-phase path: shape groups longest first onto the
    // least loaded lane (by NS flops), whole.  With the chain, everything runs
    // on the caller's stream (the chain fills the GPU by itself).
    {
        std::vector<std::pair<double, int>> work;
        for (int g = 0; g < ngroups; ++g) work.push_back({ns_flops_per_iter(p.groups[g]) * p.groups[g].count, g});
        std::sort(work.begin(), work.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
        const int lanes = S.chain ? 1 : kLanes;
        std::vector<double> load(lanes, 0.0);
        for (const auto& wg : work) {
            const int g = wg.second;
            const int l = (int)(std::min_element(load.begin(), load.end()) - load.begin());
            S.parts.push_back({g, 0, p.groups[g].count, l});
            load[l] += wg.first;
        }
    }
    S.nlanes = 1;
    for (const Part& pt : S.parts) S.nlanes = std::max(S.nlanes, pt.lane + 1);
    std::vector<int> tensor_lane(n, 0);
    for (const Part& pt : S.parts)
        for (int sl = pt.s0; sl < pt.s1; ++sl) tensor_lane[p.members[pt.group][sl]] = pt.lane;
    S.mine.assign(S.nlanes, {});
    S.legacy.assign(S.nlanes, {});
    for (int i = 0; i < n; ++i) {
        S.mine[tensor_lane[i]].push_back(i);
        if (!in_chain[p.group_of[i]]) S.legacy[tensor_lane[i]].push_back(i);
    }
    // launch sets of the per-phase path: (lane, compensated?, up to kMaxGroups parts)
    for (int l = 0; l < S.nlanes; ++l)
        for (int comp = 0; comp < 2; ++comp) {
            std::vector<int> pl;
            for (int q = 0; q < (int)S.parts.size(); ++q)
                if (S.parts[q].lane == l && (int)p.groups[S.parts[q].group].comp == comp && !in_chain[S.parts[q].group])
                    pl.push_back(q);
            for (size_t q0 = 0; q0 < pl.size(); q0 += kMaxGroups)
                S.sets.push_back({l, comp, std::vector<int>(pl.begin() + q0, pl.begin() + std::min(pl.size(), q0 + kMaxGroups))});
        }
    for (const NsLaunchSet& ls : S.sets) {
        int cnt = 0;
        for (int q : ls.parts) cnt += S.parts[q].s1 - S.parts[q].s0;
        S.max_set_count = std::max(S.max_set_count, cnt);
    }

    // ---- chain launches: each matrix bound to an XCD (longest first onto the
    // least loaded XCD by NS flops), records ordered by XCD and, within an XCD,
    // by decreasing work (the scheduler's priority)
    if (S.chain) {
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        ChainMat* recs = reinterpret_cast<ChainMat*>(ws + p.chain_rec_base);
        uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + p.chain_ctr_base);
        const size_t xe = 2;
        std::vector<ChainMat> all;
        int ctr_words = 0;
        for (const auto& lg : p.chain_launch_groups) {
            ChainLaunch L;
            memset(&L.a, 0, sizeof(L.a));
            struct M { double w; int group_idx, slot; };
            std::vector<M> mats;
            for (int gi = 0; gi < (int)lg.size(); ++gi) {
                const Group& G = p.groups[lg[gi]];
                NsGroup& D = L.a.g[gi];
                for (int b = 0; b < 2; ++b) {
                    D.x[b] = ws + G.x_off[b];
                    D.xl[b] = ws + G.xl_off[b];
                }
                D.a_hi = ws + G.ah_off;
                D.a_lo = ws + G.al_off;
                D.b = ws + G.b_off;
                D.b_lo = ws + G.bl_off;
                D.scale = reinterpret_cast<float*>(ws + p.scale_base) + G.scale_begin;
                D.count = G.count;
                D.M = G.M;
                D.N = G.N;
                for (int sl = 0; sl < G.count; ++sl) mats.push_back({ns_flops_per_iter(G), gi, sl});
            }
            (void)xe;
            std::stable_sort(mats.begin(), mats.end(), [](const M& x, const M& y) { return x.w > y.w; });
            std::vector<double> load(kXcds, 0.0);
            std::vector<std::vector<M>> per(kXcds);
            for (const M& m : mats) {
                const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
                per[x].push_back(m);
                load[x] += m.w;
            }
            L.a.mats = recs + all.size();
            L.a.ctr = ctr + ctr_words;
            L.a.rowsq = reinterpret_cast<const float*>(ws + p.rowsq_base);
            int nm = 0;
            for (int x = 0; x < kXcds; ++x) {
                L.a.xcd_begin[x] = nm;
                for (const M& m : per[x]) {
                    const int gidx = lg[m.group_idx];
                    const Group& G = p.groups[gidx];
                    const int ti = p.members[gidx][m.slot];
                    const muon_tensor_t& t = tensors[ti];
                    ChainMat R;
                    memset(&R, 0, sizeof(R));
                    R.param = t.param;
                    R.out = t.update_out;
                    R.ema = t.ema;
                    R.shape_scale = shape_scale_of(t);
                    R.flags = (t.rows > t.cols ? kApplyTransposed : 0) | (vec_ok(t) ? kApplyVec : 0);
                    R.rows = t.rows;
                    R.cols = t.cols;
                    R.group = m.group_idx;
                    R.slot = m.slot;
                    R.rowsq_off = (int)p.rowsq_off[ti];
                    const int tm = G.M / kTile, tn = G.N / kTile;
                    R.tiles_sym = tm * (tm + 1) / 2;
                    R.tiles_upd = tm * tn;
                    all.push_back(R);
                    ++nm;
                }
            }
            L.a.xcd_begin[kXcds] = nm;
            L.a.nmat = nm;
            L.a.timeout_ticks = (uint64_t)100000000 * 10;   // 10 s of the 100 MHz counter
            ctr_words += (nm + 1) * kChainCtrWords;         // counters, then the launch's status block
            S.chains.push_back(L);
        }
        for (size_t r0 = 0; r0 < all.size(); r0 += kChainSetupChunk) {
            ChainSetupArgs sa;
            memset(&sa, 0, sizeof(sa));
            sa.n = (int)std::min(all.size() - r0, (size_t)kChainSetupChunk);
            for (int i = 0; i < sa.n; ++i) sa.rec[i] = all[r0 + i];
            sa.dst = recs + r0;
            if (r0 == 0) {
                sa.zero = ctr;
                sa.nzero = ctr_words;
            }
            S.setups.push_back(sa);
        }
    }
    return MUON_OK;
}

// The cached schedule of this signature, or a new one; null on a validation
// error (its code in rc).
std::shared_ptr<Schedule> find_schedule(const muon_tensor_t* t, int n, int mode, void* ws, size_t ws_bytes, int& rc) {
    rc = MUON_OK;
    const int schedule = g_ns_schedule.load();
    std::vector<uint64_t> key = schedule_key(t, n, mode, schedule, ws, ws_bytes);
    {
        std::lock_guard<std::mutex> lk(g_sched_mu);
        for (size_t i = 0; i < g_sched.size(); ++i)
            if (g_sched[i]->key == key) {
                std::shared_ptr<Schedule> hit = g_sched[i];
                g_sched.erase(g_sched.begin() + i);
                g_sched.push_back(hit);
                ++g_sched_hits;
                return hit;
            }
    }
    auto S = std::make_shared<Schedule>();
    rc = build_schedule(t, n, mode, schedule, ws, ws_bytes, *S);
    if (rc != MUON_OK) return nullptr;
    S->key = std::move(key);
    std::lock_guard<std::mutex> lk(g_sched_mu);
    ++g_sched_built;
    g_sched.push_back(S);
    if (g_sched.size() > kMaxSchedules) g_sched.erase(g_sched.begin());
    return S;
}


// ------------------------------------------------------------- static workspace
// The allocation-free entry point's workspace: a file-scope device array that
// every GPU the library runs on holds until the process ends.  Host code never
// uses the array's name as an address: its device address comes from
// hipGetSymbolAddress, once per device, and is kept here.
constexpr size_t kStaticScratchBytes = MUON_STATIC_WORKSPACE_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

int static_scratch(void*& out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr)
            return fail(MUON_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(err));
        it = g_scratch_ptr.emplace(dev, ptr).first;
    }
    out = it->second;
    return MUON_OK;
}

// ------------------------------------------------------------- EMA lists
// Arguments of an EMA list (ema_update, muon_step_ema): non-NULL arrays,
// 1 <= n <= MUON_MAX_TENSORS, element counts in [0, kMaxStreamElems], 4-byte
// aligned non-NULL buffers for every non-empty tensor.  The byte spans of the
// buffers are appended to `spans` (tensor ids 0 .. n-1) for the caller's
// overlap check.
int validate_ema_list(float* const* ema, const float* const* params, const int64_t* numel, int32_t n,
                      std::vector<Span>& spans) {
    if (!ema || !params || !numel) return fail(MUON_ERR_INVALID_ARG, "ema, params and numel must be non-NULL");
    if (n <= 0 || n > MUON_MAX_TENSORS) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, MUON_MAX_TENSORS);
    for (int i = 0; i < n; ++i) {
        if (numel[i] < 0) return fail(MUON_ERR_INVALID_ARG, "numel[%d] = %lld is negative", i, (long long)numel[i]);
        if (numel[i] > kMaxStreamElems)
            return fail(MUON_ERR_UNSUPPORTED, "numel[%d] = %lld beyond %lld", i, (long long)numel[i],
                        (long long)kMaxStreamElems);
        if (numel[i] == 0) continue;
        if (!ema[i] || !params[i]) return fail(MUON_ERR_INVALID_ARG, "tensor %d: NULL pointer", i);
        if (reinterpret_cast<uintptr_t>(ema[i]) % 4 || reinterpret_cast<uintptr_t>(params[i]) % 4)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: pointer not 4-byte aligned", i);
        const uintptr_t e = reinterpret_cast<uintptr_t>(ema[i]);
        const uintptr_t q = reinterpret_cast<uintptr_t>(params[i]);
        const size_t bytes = (size_t)numel[i] * sizeof(float);
        spans.push_back({e, e + bytes, i});
        spans.push_back({q, q + bytes, i});
    }
    return MUON_OK;
}

// The EMA kernels over a validated list: table entries of at most
// kEmaEntryElems elements, kEmaChunk per launch.
int enqueue_ema_list(float* const* ema, const float* const* params, const int64_t* numel, int32_t n, float decay,
                     hipStream_t s) {
    int i = 0;
    int64_t off = 0;
    while (i < n) {
        EmaArgs a;
        memset(&a, 0, sizeof(a));
        a.decay = decay;
        a.one_minus_decay = 1.0f - decay;
        int64_t blocks = 0;
        while (i < n && a.n < kEmaChunk) {
            if (off >= numel[i]) { ++i; off = 0; continue; }
            const int64_t len = std::min(numel[i] - off, kEmaEntryElems);
            const int64_t nb = (len + kEmaElemsPerBlock - 1) / kEmaElemsPerBlock;
            if (blocks + nb > (int64_t)1 << 30) break;
            EmaTensor& T = a.t[a.n++];
            T.ema = ema[i] + off;
            T.param = params[i] + off;
            T.numel = (int)len;
            T.block_begin = (int)blocks;
            blocks += nb;
            off += len;
        }
        if (a.n == 0) continue;
        hipError_t err = timed_launch("ema", s, [&] { return launch_ema(a, (int)blocks, s); });
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "ema launch failed: %s", hipGetErrorString(err));
    }
    return MUON_OK;
}

// The other parameters' weight EMA that muon_step_ema runs with the step.
struct EmaList {
    float* const* ema;
    const float* const* params;
    const int64_t* numel;
    int32_t n;
};

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

const char* muon_last_error(void) { return g_last_error.c_str(); }

int muon_version(void) { return 10000; }

size_t muon_workspace_size(const muon_tensor_t* tensors, int32_t n, int32_t ns_precision) {
    if (validate_tensors(tensors, n, ns_precision) != MUON_OK) return 0;
    Plan p;
    make_plan(tensors, n, ns_precision, p);
    return p.bytes;
}

// muon_step, and with `extra` the weight EMA of further tensors enqueued on the
// lightest lane once its matrices are done (muon_step_ema).  Every argument has
// been or is validated before anything is enqueued.
static int muon_step_impl(const muon_tensor_t* tensors, int32_t n, float lr, float momentum, int32_t nesterov,
                          float weight_decay, int32_t row_norm, int32_t ns_steps, const float* ns_coeffs,
                          int32_t ns_precision, float ema_decay, const EmaList* extra, void* workspace,
                          size_t workspace_bytes, void* stream) {
    int rc = validate_tensors(tensors, n, ns_precision);
    if (rc) return rc;
    if (!std::isfinite(lr) || !std::isfinite(momentum) || !std::isfinite(weight_decay))
        return fail(MUON_ERR_INVALID_ARG, "lr, momentum and weight_decay must be finite");
    if (!std::isfinite(ema_decay) || ema_decay < 0.f || ema_decay > 1.f)
        return fail(MUON_ERR_INVALID_ARG, "ema_decay must be finite and in [0, 1]");
    if ((nesterov != 0 && nesterov != 1) || (row_norm != 0 && row_norm != 1))
        return fail(MUON_ERR_INVALID_ARG, "nesterov and row_norm must be 0 or 1");
    if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS)
        return fail(MUON_ERR_INVALID_ARG, "ns_steps = %d outside [0, %d]", ns_steps, MUON_MAX_NS_STEPS);
    if (ns_steps > 0 && !ns_coeffs) return fail(MUON_ERR_INVALID_ARG, "ns_coeffs is NULL with ns_steps = %d", ns_steps);
    for (int k = 0; k < 3 * ns_steps; ++k)
        if (!std::isfinite(ns_coeffs[k])) return fail(MUON_ERR_INVALID_ARG, "ns_coeffs[%d] is not finite", k);
    std::shared_ptr<Schedule> sched = find_schedule(tensors, n, ns_precision, workspace, workspace_bytes, rc);
    if (!sched) return rc;
    const Schedule& S = *sched;
    const Plan& p = S.p;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* rowsq = reinterpret_cast<float*>(ws + p.rowsq_base);
    const int prec = S.prec;                                             // storage precision
    const size_t xe = prec == kNsBf16 ? 2 : 4;                           // bytes per X element
    // bytes per element of X's lo plane: base-precision bf16 groups keep bytes
    // (the NS kernels index that plane by element), the compensated ones bf16
    auto lo_bytes = [&](const Group& G) -> size_t { return prec == kNsBf16 ? (G.comp ? 2 : 1) : xe; };
    hipError_t err = hipSuccess;
    // the chain runs the NS iterations of its groups; with no iteration every
    // matrix takes the per-phase path's prep, Frobenius scale and apply
    const bool use_chain = S.chain && ns_steps > 0;
    const std::vector<std::vector<int>>& legacy = use_chain ? S.legacy : S.mine;
    const int nlanes = S.nlanes;
    const std::vector<Part>& parts = S.parts;

    // The weight update runs inside the last NS update launch when every launch
    // holds at most kMaxFused matrices.  The first Gram launch computes the
    // Frobenius scales itself (no separate frob launch) when every launch holds
    // at most kMaxFrobSlots matrices.
    const bool fuse = ns_steps > 0 && S.max_set_count <= kMaxFused;
    const bool fold_frob = ns_steps > 0 && S.max_set_count <= kMaxFrobSlots;
    const float keep = 1.0f - lr * weight_decay;
    // e4m3 scale exponents of the table (cached per thread for the last table)
    thread_local std::vector<float> f8_last;
    thread_local int f8_sa[MUON_MAX_NS_STEPS];
    if (f8_last.size() != (size_t)(3 * ns_steps) ||
        (ns_steps > 0 && memcmp(f8_last.data(), ns_coeffs, sizeof(float) * 3 * ns_steps) != 0)) {
        f8_scale_exponents(ns_coeffs, ns_steps, f8_sa);
        f8_last.assign(ns_coeffs, ns_coeffs + 3 * ns_steps);
    }
    auto lr_scale = [&](const muon_tensor_t& x) { return lr * shape_scale_of(x); };

    std::unique_lock<std::mutex> lane_lock(g_lane_mu, std::defer_lock);
    hipStream_t lane_stream[kLanes];
    for (int l = 0; l < kLanes; ++l) lane_stream[l] = s;
    LaneSet* L = nullptr;
    if (nlanes > 1) {
        lane_lock.lock();
        int dev = 0;
        err = hipGetDevice(&dev);
        if (err == hipSuccess) err = lanes_for_device(dev, L);
        if (err == hipSuccess) err = hipEventRecord(L->fork, s);
        for (int l = 1; l < nlanes && err == hipSuccess; ++l) {
            lane_stream[l] = L->stream[l];
            err = hipStreamWaitEvent(lane_stream[l], L->fork, 0);
        }
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "lane fork failed: %s", hipGetErrorString(err));
    }

    // ---- chain records and counters (before prep: nothing waits for it)
    if (use_chain) {
        for (const ChainSetupArgs& sa : S.setups) {
            err = timed_launch("chain_setup", s, [&] { return launch_chain_setup(sa, s); });
            if (err != hipSuccess) return fail(MUON_ERR_HIP, "chain setup launch failed: %s", hipGetErrorString(err));
        }
    }

    // ---- prep: momentum, row norm, X0 (short side first, zero padded), in
    // evenly sized launches of at most kPrepChunk tensors
    auto enqueue_prep = [&](int lane) -> int {
        hipStream_t ls_stream = lane_stream[lane];
        const std::vector<int>& my = S.mine[lane];
        const int nm = (int)my.size();
        const int prep_launches = (nm + kPrepChunk - 1) / kPrepChunk;
        const int prep_take = (nm + prep_launches - 1) / prep_launches;
        for (int c0 = 0; c0 < nm;) {
            PrepArgs a;
            memset(&a, 0, sizeof(a));
            a.mu = momentum;
            a.nesterov = nesterov;
            a.row_norm = row_norm;
            int blocks = 0;
            size_t lds = 0;
            for (int k = 0; k < prep_take && c0 < nm; ++k, ++c0) {
                const int i = my[c0];
                const muon_tensor_t& x = tensors[i];
                const Group& G = p.groups[p.group_of[i]];
                PrepTensor& T = a.t[a.n++];
                T.grad = x.grad;
                T.mom = x.momentum;
                const size_t slot_off = (size_t)p.slot_of[i] * G.M * G.N * xe;
                T.xh = ws + G.x_off[0] + slot_off;
                T.xl = ws + G.xl_off[0] + (size_t)p.slot_of[i] * G.M * G.N * lo_bytes(G);
                T.rowsq = rowsq + p.rowsq_off[i];
                T.rows = x.rows;
                T.cols = x.cols;
                T.transposed = x.rows > x.cols;
                T.m_pad = G.M;
                T.n_pad = G.N;
                T.vec = (x.cols % 4 == 0) && (reinterpret_cast<uintptr_t>(x.grad) % 16 == 0) &&
                        (reinterpret_cast<uintptr_t>(x.momentum) % 16 == 0);
                T.lo8 = prec == kNsBf16 && !G.comp;
                T.block_begin = blocks;
                if (T.transposed) {
                    T.rb = transposed_rb(x.cols);
                    blocks += G.N / T.rb;
                    lds = std::max(lds, (size_t)T.rb * (x.cols + 1) * sizeof(float));
                } else {
                    T.rb = kRowsPerWaveBlock;
                    blocks += G.M / kRowsPerWaveBlock;
                }
            }
            err = timed_launch("prep", ls_stream, [&] { return launch_prep(a, prec, blocks, lds, ls_stream); });
            if (err != hipSuccess) return fail(MUON_ERR_HIP, "prep launch failed: %s", hipGetErrorString(err));
        }
        return MUON_OK;
    };

    // ---- Frobenius scales (per-phase path)
    auto enqueue_frob = [&](int lane) -> int {
        hipStream_t ls_stream = lane_stream[lane];
        const std::vector<int>& my = legacy[lane];
        const int nm = (int)my.size();
        for (int c0 = 0; c0 < nm; c0 += kFrobChunk) {
            FrobArgs a;
            memset(&a, 0, sizeof(a));
            a.rowsq = rowsq;
            a.scale = reinterpret_cast<float*>(ws + p.scale_base);
            for (int c = c0; c < std::min(nm, c0 + kFrobChunk); ++c) {
                const int i = my[c];
                const Group& G = p.groups[p.group_of[i]];
                a.rowsq_off[a.n] = (int)p.rowsq_off[i];
                a.rows[a.n] = tensors[i].rows;
                a.scale_idx[a.n] = G.scale_begin + p.slot_of[i];
                ++a.n;
            }
            err = timed_launch("frob", ls_stream, [&] { return launch_frob(a, ls_stream); });
            if (err != hipSuccess) return fail(MUON_ERR_HIP, "frob launch failed: %s", hipGetErrorString(err));
        }
        return MUON_OK;
    };

    // ---- one Newton-Schulz phase of iteration k: one launch per launch set
    auto enqueue_ns = [&](int lane, int k, int phase) -> int {
        hipStream_t ls_stream = lane_stream[lane];
        for (const NsLaunchSet& ls : S.sets) {
            if (ls.lane != lane) continue;
            NsArgs a;
            memset(&a, 0, sizeof(a));
            a.src = k & 1;
            a.first = (k == 0);
            a.a = ns_coeffs[3 * k + 0];
            a.b = ns_coeffs[3 * k + 1];
            a.c = ns_coeffs[3 * k + 2];
            a.fuse_apply = fuse && phase == kUpdate && k == ns_steps - 1;
            a.keep = keep;
            a.decay = ema_decay;
            a.one_minus_decay = 1.0f - ema_decay;
            a.fold_frob = fold_frob && phase == kGram && k == 0;
            a.rowsq = rowsq;
            a.f8_sa = f8_sa[k];
            a.f8_sl = f8_sa[k] + 8;
            int jobs = 0, napply = 0, nfrob = 0;
            for (int q : ls.parts) {
                const Part& pt = parts[q];
                const Group& G = p.groups[pt.group];
                const int count = pt.s1 - pt.s0;
                const size_t xslot = (size_t)G.M * G.N * xe, aslot = (size_t)G.M * G.M * xe;
                NsGroup& D = a.g[a.ngroups++];
                for (int b = 0; b < 2; ++b) {
                    D.x[b] = ws + G.x_off[b] + pt.s0 * xslot;
                    D.xl[b] = ws + G.xl_off[b] + pt.s0 * (size_t)G.M * G.N * lo_bytes(G);
                }
                D.a_hi = ws + G.ah_off + pt.s0 * aslot;
                D.a_lo = ws + G.al_off + pt.s0 * aslot;
                D.b = ws + G.b_off + pt.s0 * aslot;
                D.b_lo = ws + G.bl_off + pt.s0 * aslot;
                D.scale = reinterpret_cast<float*>(ws + p.scale_base) + G.scale_begin + pt.s0;
                D.count = count;
                D.M = G.M;
                D.N = G.N;
                D.job_begin = jobs;
                D.apply_begin = napply;
                D.frob_begin = nfrob;
                if (a.fold_frob) {
                    for (int sl = pt.s0; sl < pt.s1; ++sl) {
                        const int ti = p.members[pt.group][sl];
                        a.frob[nfrob++] = {(int)p.rowsq_off[ti], tensors[ti].rows};
                    }
                }
                if (a.fuse_apply) {
                    for (int sl = pt.s0; sl < pt.s1; ++sl) {
                        const int ti = p.members[pt.group][sl];
                        const muon_tensor_t& x = tensors[ti];
                        FusedApply& F = a.apply[napply++];
                        F.param = x.param;
                        F.out = x.update_out;
                        F.ema = x.ema;
                        F.rows = x.rows;
                        F.cols = x.cols;
                        F.flags = (x.rows > x.cols ? kApplyTransposed : 0) | (vec_ok(x) ? kApplyVec : 0);
                        F.lr_s = lr_scale(x);
                    }
                }
                const int tm = G.M / kTile, tn = G.N / kTile;
                jobs += count * (phase == kUpdate ? tm * tn : tm * (tm + 1) / 2);
            }
            a.total_jobs = jobs;
            const bool comp = ls.comp != 0;
            const char* name = ns_kernel_name(phase, prec, comp, a.fuse_apply != 0);
            err = timed_launch(name, ls_stream, [&] { return launch_ns(a, phase, prec, comp, ls_stream); });
            if (err != hipSuccess) return fail(MUON_ERR_HIP, "%s launch failed: %s", name, hipGetErrorString(err));
        }
        return MUON_OK;
    };

    // ---- apply: W' = (1 - lr wd) W - lr s O and the EMA (unless the last NS
    // update did it)
    auto enqueue_apply = [&](int lane) -> int {
        hipStream_t ls_stream = lane_stream[lane];
        const std::vector<int>& my = legacy[lane];
        const int nm = (int)my.size();
        const int final_buf = ns_steps & 1;
        for (int c0 = 0; c0 < nm; c0 += kApplyChunk) {
            ApplyArgs a;
            memset(&a, 0, sizeof(a));
            a.keep = keep;
            a.decay = ema_decay;
            a.one_minus_decay = 1.0f - ema_decay;
            a.use_scale = ns_steps == 0;
            int blocks = 0;
            size_t lds = 0;
            for (int c = c0; c < std::min(nm, c0 + kApplyChunk); ++c) {
                const int i = my[c];
                const muon_tensor_t& x = tensors[i];
                const Group& G = p.groups[p.group_of[i]];
                ApplyTensor& T = a.t[a.n++];
                T.param = x.param;
                T.out = x.update_out;
                T.ema = x.ema;
                const size_t slot_off = (size_t)p.slot_of[i] * G.M * G.N * xe;
                T.xh = ws + G.x_off[final_buf] + slot_off;
                T.xl = ws + G.xl_off[final_buf] + (size_t)p.slot_of[i] * G.M * G.N * lo_bytes(G);
                T.scale = reinterpret_cast<const float*>(ws + p.scale_base) + G.scale_begin + p.slot_of[i];
                T.lr_s = lr_scale(x);
                T.rows = x.rows;
                T.cols = x.cols;
                T.n_pad = G.N;
                T.transposed = x.rows > x.cols;
                T.vec = vec_ok(x);
                T.lo8 = prec == kNsBf16 && !G.comp;
                T.block_begin = blocks;
                if (T.transposed) {
                    T.rb = transposed_rb(x.cols);
                    blocks += (x.rows + T.rb - 1) / T.rb;
                    lds = std::max(lds, (size_t)T.rb * (x.cols + 1) * sizeof(float));
                } else {
                    T.rb = kRowsPerWaveBlock;
                    blocks += (x.rows + kRowsPerWaveBlock - 1) / kRowsPerWaveBlock;
                }
            }
            err = timed_launch("apply", ls_stream, [&] { return launch_apply(a, prec, blocks, lds, ls_stream); });
            if (err != hipSuccess) return fail(MUON_ERR_HIP, "apply launch failed: %s", hipGetErrorString(err));
        }
        return MUON_OK;
    };

    // ---- the chain: every NS iteration of its groups in one launch per chunk
    // of kMaxGroups groups, on the caller's stream
    auto enqueue_chain = [&]() -> int {
        int dev = 0;
        err = hipGetDevice(&dev);
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
        const int cus = device_cus(dev);
        const int wgs = std::max(cus, kXcds) * kChainWgPerCu;
        for (const ChainLaunch& CL : S.chains) {
            ChainArgs a = CL.a;
            a.ns_steps = ns_steps;
            a.fuse_apply = 1;
            a.keep = keep;
            a.lr = lr;
            a.decay = ema_decay;
            a.one_minus_decay = 1.0f - ema_decay;
            for (int k = 0; k < ns_steps; ++k) {
                a.a[k] = ns_coeffs[3 * k + 0];
                a.b[k] = ns_coeffs[3 * k + 1];
                a.c[k] = ns_coeffs[3 * k + 2];
                a.f8_sa[k] = f8_sa[k];
            }
            err = timed_launch("ns_chain_bf16", s, [&] { return launch_chain(a, wgs, s); });
            if (err != hipSuccess) return fail(MUON_ERR_HIP, "ns_chain launch failed: %s", hipGetErrorString(err));
        }
        return MUON_OK;
    };

    // Enqueue stage by stage across the lanes, so every lane has work queued
    // early even when the host is only just ahead of the GPU.
    for (int lane = 0; lane < nlanes; ++lane)
        if ((rc = enqueue_prep(lane))) return rc;
    if (!fold_frob)
        for (int lane = 0; lane < nlanes; ++lane)
            if ((rc = enqueue_frob(lane))) return rc;
    for (int k = 0; k < ns_steps; ++k)
        for (int phase = kGram; phase <= kUpdate; ++phase)
            for (int lane = 0; lane < nlanes; ++lane)
                if ((rc = enqueue_ns(lane, k, phase))) return rc;
    if (!fuse)
        for (int lane = 0; lane < nlanes; ++lane)
            if ((rc = enqueue_apply(lane))) return rc;
    if (use_chain && (rc = enqueue_chain())) return rc;
    // the other parameters' EMA: its tensors are disjoint from the matrices,
    // so it runs on the lane with the least NS work, beside the others' last
    // phases, instead of after the join
    if (extra && (rc = enqueue_ema_list(extra->ema, extra->params, extra->numel, extra->n, ema_decay,
                                        lane_stream[nlanes - 1])))
        return rc;

    if (L) {
        for (int l = 1; l < nlanes && err == hipSuccess; ++l) {
            err = hipEventRecord(L->join[l], lane_stream[l]);
            if (err == hipSuccess) err = hipStreamWaitEvent(s, L->join[l], 0);
        }
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "lane join failed: %s", hipGetErrorString(err));
    }
    return MUON_OK;
}

int muon_step(const muon_tensor_t* tensors, int32_t n, float lr, float momentum, int32_t nesterov,
              float weight_decay, int32_t row_norm, int32_t ns_steps, const float* ns_coeffs,
              int32_t ns_precision, float ema_decay, void* workspace, size_t workspace_bytes, void* stream) {
    return muon_step_impl(tensors, n, lr, momentum, nesterov, weight_decay, row_norm, ns_steps, ns_coeffs,
                          ns_precision, ema_decay, nullptr, workspace, workspace_bytes, stream);
}

int muon_step_ema(const muon_tensor_t* tensors, int32_t n, float lr, float momentum, int32_t nesterov,
                  float weight_decay, int32_t row_norm, int32_t ns_steps, const float* ns_coeffs,
                  int32_t ns_precision, float ema_decay, float* const* extra_ema, const float* const* extra_params,
                  const int64_t* extra_numel, int32_t n_extra, void* workspace, size_t workspace_bytes,
                  void* stream) {
    int rc = validate_tensors(tensors, n, ns_precision);
    if (rc) return rc;
    if (n_extra == 0)
        return muon_step_impl(tensors, n, lr, momentum, nesterov, weight_decay, row_norm, ns_steps, ns_coeffs,
                              ns_precision, ema_decay, nullptr, workspace, workspace_bytes, stream);
    // the extra list, and no overlap between its buffers, the matrices' buffers
    // and the workspace (ids: extra tensors 0 .. n_extra-1, then the matrices)
    std::vector<Span> spans;
    if ((rc = validate_ema_list(extra_ema, extra_params, extra_numel, n_extra, spans))) return rc;
    for (int i = 0; i < n; ++i) {
        const muon_tensor_t& x = tensors[i];
        const size_t bytes = (size_t)x.rows * x.cols * sizeof(float);
        const void* ptrs[5] = {x.param, x.grad, x.momentum, x.update_out, x.ema};
        for (int k = 0; k < 5; ++k) {
            if (!ptrs[k]) continue;
            const uintptr_t lo = reinterpret_cast<uintptr_t>(ptrs[k]);
            spans.push_back({lo, lo + bytes, n_extra + i});
        }
    }
    if (workspace && workspace_bytes) {
        const uintptr_t w = reinterpret_cast<uintptr_t>(workspace);
        spans.push_back({w, w + workspace_bytes, n_extra + n});
    }
    if ((rc = check_overlaps(spans, "muon_step_ema"))) return rc;
    const EmaList extra{extra_ema, extra_params, extra_numel, n_extra};
    return muon_step_impl(tensors, n, lr, momentum, nesterov, weight_decay, row_norm, ns_steps, ns_coeffs,
                          ns_precision, ema_decay, &extra, workspace, workspace_bytes, stream);
}

int muon_step_static(const muon_tensor_t* tensors, int32_t n, float lr, float momentum, int32_t nesterov,
                     float weight_decay, int32_t row_norm, int32_t ns_steps, const float* ns_coeffs,
                     int32_t ns_precision, float ema_decay, void* stream) {
    int rc = validate_tensors(tensors, n, ns_precision);
    if (rc) return rc;
    Plan p;
    make_plan(tensors, n, ns_precision, p);
    if (p.bytes > kStaticScratchBytes)
        return fail(MUON_ERR_WORKSPACE,
                    "these matrices need %zu bytes of workspace; the static workspace holds %zu (use muon_step with "
                    "a caller workspace)", p.bytes, kStaticScratchBytes);
    void* ws = nullptr;
    if ((rc = static_scratch(ws))) return rc;
    return muon_step(tensors, n, lr, momentum, nesterov, weight_decay, row_norm, ns_steps, ns_coeffs, ns_precision,
                     ema_decay, ws, kStaticScratchBytes, stream);
}

int muon_set_ns_schedule(int32_t schedule) {
    if (schedule != MUON_NS_SCHEDULE_PHASES && schedule != MUON_NS_SCHEDULE_CHAIN)
        return fail(MUON_ERR_INVALID_ARG, "schedule = %d is not MUON_NS_SCHEDULE_PHASES or MUON_NS_SCHEDULE_CHAIN",
                    schedule);
    return g_ns_schedule.exchange(schedule);
}

int muon_plan_cache_stats(int64_t* built, int64_t* hits) {
    std::lock_guard<std::mutex> lk(g_sched_mu);
    if (built) *built = g_sched_built;
    if (hits) *hits = g_sched_hits;
    return (int)g_sched.size();
}

int ema_update(float* const* ema, const float* const* params, const int64_t* numel, int32_t n, float decay,
               void* stream) {
    if (!std::isfinite(decay) || decay < 0.f || decay > 1.f)
        return fail(MUON_ERR_INVALID_ARG, "decay must be finite and in [0, 1]");
    std::vector<Span> spans;
    int rc = validate_ema_list(ema, params, numel, n, spans);
    if (rc) return rc;
    // no two buffers of the call may overlap
    if ((rc = check_overlaps(spans, "ema_update"))) return rc;
    return enqueue_ema_list(ema, params, numel, n, decay, static_cast<hipStream_t>(stream));
}

int ema_swap(float* const* ema, float* const* params, const int64_t* numel, int32_t n, void* stream) {
    if (!ema || !params || !numel) return fail(MUON_ERR_INVALID_ARG, "ema, params and numel must be non-NULL");
    if (n <= 0 || n > MUON_MAX_TENSORS) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, MUON_MAX_TENSORS);
    std::vector<Span> spans;
    for (int i = 0; i < n; ++i) {
        if (numel[i] < 0) return fail(MUON_ERR_INVALID_ARG, "numel[%d] = %lld is negative", i, (long long)numel[i]);
        if (numel[i] > kMaxStreamElems)
            return fail(MUON_ERR_UNSUPPORTED, "numel[%d] = %lld beyond %lld", i, (long long)numel[i],
                        (long long)kMaxStreamElems);
        if (numel[i] == 0) continue;
        if (!ema[i] || !params[i]) return fail(MUON_ERR_INVALID_ARG, "tensor %d: NULL pointer", i);
        if (reinterpret_cast<uintptr_t>(ema[i]) % 4 || reinterpret_cast<uintptr_t>(params[i]) % 4)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: pointer not 4-byte aligned", i);
        const uintptr_t e = reinterpret_cast<uintptr_t>(ema[i]);
        const uintptr_t q = reinterpret_cast<uintptr_t>(params[i]);
        const size_t bytes = (size_t)numel[i] * sizeof(float);
        spans.push_back({e, e + bytes, i});
        spans.push_back({q, q + bytes, i});
    }
    int rc = check_overlaps(spans, "ema_swap");
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // table entries of at most kEmaEntryElems elements, kEmaChunk per launch
    int i = 0;
    int64_t off = 0;
    while (i < n) {
        SwapArgs a;
        memset(&a, 0, sizeof(a));
        int64_t blocks = 0;
        while (i < n && a.n < kEmaChunk) {
            if (off >= numel[i]) { ++i; off = 0; continue; }
            const int64_t len = std::min(numel[i] - off, kEmaEntryElems);
            const int64_t nb = (len + kEmaElemsPerBlock - 1) / kEmaElemsPerBlock;
            if (blocks + nb > (int64_t)1 << 30) break;
            SwapTensor& T = a.t[a.n++];
            T.a = ema[i] + off;
            T.b = params[i] + off;
            T.numel = (int)len;
            T.block_begin = (int)blocks;
            blocks += nb;
            off += len;
        }
        if (a.n == 0) continue;
        hipError_t err = timed_launch("swap", s, [&] { return launch_swap(a, (int)blocks, s); });
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "swap launch failed: %s", hipGetErrorString(err));
    }
    return MUON_OK;
}

int adamw_step(const adamw_tensor_t* tensors, int32_t n, float lr, float beta1, float beta2, float eps,
               float weight_decay, int32_t step, float ema_decay, void* stream) {
    if (!tensors) return fail(MUON_ERR_INVALID_ARG, "tensors is NULL");
    if (n <= 0 || n > MUON_MAX_TENSORS) return fail(MUON_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, MUON_MAX_TENSORS);
    if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(eps))
        return fail(MUON_ERR_INVALID_ARG, "lr, weight_decay and eps must be finite");
    if (eps < 0.f) return fail(MUON_ERR_INVALID_ARG, "eps must be >= 0");
    if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
        return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must be in [0, 1)");
    if (step < 1) return fail(MUON_ERR_INVALID_ARG, "step = %d must be >= 1", step);
    if (!std::isfinite(ema_decay) || ema_decay < 0.f || ema_decay > 1.f)
        return fail(MUON_ERR_INVALID_ARG, "ema_decay must be finite and in [0, 1]");
    std::vector<Span> spans;
    for (int i = 0; i < n; ++i) {
        const adamw_tensor_t& x = tensors[i];
        if (x.numel < 0) return fail(MUON_ERR_INVALID_ARG, "tensor %d: numel = %lld is negative", i, (long long)x.numel);
        if (x.numel > kMaxStreamElems)
            return fail(MUON_ERR_UNSUPPORTED, "tensor %d: numel = %lld beyond %lld", i, (long long)x.numel,
                        (long long)kMaxStreamElems);
        if (x.numel == 0) continue;
        if (!x.param || !x.grad || !x.exp_avg || !x.exp_avg_sq)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: param, grad, exp_avg and exp_avg_sq must be non-NULL", i);
        const void* ptrs[5] = {x.param, x.grad, x.exp_avg, x.exp_avg_sq, x.ema};
        const size_t bytes = (size_t)x.numel * sizeof(float);
        for (int k = 0; k < 5; ++k) {
            if (!ptrs[k]) continue;
            const uintptr_t lo = reinterpret_cast<uintptr_t>(ptrs[k]);
            if (lo % sizeof(float)) return fail(MUON_ERR_INVALID_ARG, "tensor %d: pointer %d is not 4-byte aligned", i, k);
            spans.push_back({lo, lo + bytes, i});
        }
    }
    int rc = check_overlaps(spans, "adamw_step");
    if (rc) return rc;
    // bias corrections in double, folded into two fp32 factors
    const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
    const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int i = 0;
    while (i < n) {
        AdamArgs a;
        memset(&a, 0, sizeof(a));
        a.keep = 1.0f - lr * weight_decay;
        a.beta1 = beta1;
        a.one_minus_beta1 = 1.0f - beta1;
        a.beta2 = beta2;
        a.one_minus_beta2 = 1.0f - beta2;
        a.step_size = (float)((double)lr / bc1);
        a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
        a.eps = eps;
        a.decay = ema_decay;
        a.one_minus_decay = 1.0f - ema_decay;
        int64_t blocks = 0;
        for (; i < n && a.n < kAdamChunk; ++i) {
            const adamw_tensor_t& x = tensors[i];
            if (x.numel == 0) continue;
            const int64_t nb = (x.numel + kAdamElemsPerBlock - 1) / kAdamElemsPerBlock;
            if (blocks + nb > (int64_t)1 << 30) break;
            AdamTensor& T = a.t[a.n++];
            T.param = x.param;
            T.grad = x.grad;
            T.m = x.exp_avg;
            T.v = x.exp_avg_sq;
            T.ema = x.ema;
            T.numel = x.numel;
            T.block_begin = (int)blocks;
            T.vec = 1;
            const void* ptrs[5] = {x.param, x.grad, x.exp_avg, x.exp_avg_sq, x.ema};
            for (int k = 0; k < 5; ++k)
                if (reinterpret_cast<uintptr_t>(ptrs[k]) % 16) T.vec = 0;
            blocks += nb;
        }
        if (a.n == 0) continue;
        hipError_t err = timed_launch("adamw", s, [&] { return launch_adamw(a, (int)blocks, s); });
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "adamw launch failed: %s", hipGetErrorString(err));
    }
    return MUON_OK;
}

int muon_profile_enable(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_enabled = enable != 0;
    return MUON_OK;
}

int muon_profile_read(char* names, int64_t* counts, double* total_ms, int32_t cap, int32_t reset) {
    std::vector<PendingEvent> pending;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        pending.swap(g_pending);
    }
    for (PendingEvent& e : pending) {
        hipError_t err = hipEventSynchronize(e.stop);
        float ms = 0.f;
        if (err == hipSuccess) err = hipEventElapsedTime(&ms, e.start, e.stop);
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (err != hipSuccess) return fail(MUON_ERR_HIP, "profile event: %s", hipGetErrorString(err));
        auto it = std::find_if(g_totals.begin(), g_totals.end(), [&](const auto& kv) { return kv.first == e.name; });
        if (it == g_totals.end()) {
            g_totals.push_back({e.name, ProfileTotal()});
            it = g_totals.end() - 1;
        }
        it->second.count += 1;
        it->second.ms += ms;
        g_event_pool.push_back(e.start);
        g_event_pool.push_back(e.stop);
    }
    std::lock_guard<std::mutex> lk(g_prof_mu);
    const int total = (int)g_totals.size();
    for (int i = 0; i < total && i < cap; ++i) {
        if (names) {
            strncpy(names + 48 * i, g_totals[i].first.c_str(), 47);
            names[48 * i + 47] = '\0';
        }
        if (counts) counts[i] = g_totals[i].second.count;
        if (total_ms) total_ms[i] = g_totals[i].second.ms;
    }
    if (reset) g_totals.clear();
    return total;
}

}  // extern "C"
