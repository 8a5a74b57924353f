// conv.hip -- causal depthwise conv1d with state (prefill) and its decode-time update.
//
// Prefill, causal-conv1d tutorial ch. 7, "defining the state through the extended sequence"
// and "packed-sequence boundaries": out_t = phi(bias + sum_k w_k u_{t+k}) over
// u = [S, x]; F = u[L : L+K-1].  Each thread owns V adjacent channels of one batch row and a
// run of TT tokens; the K-1 previous inputs live in registers and slide along the run, so
// every input element is read from HBM once (plus a K-1 halo per run).  Channel-last rows
// give coalesced vector loads/stores (2 bf16 channels per thread in the bf16 kernel below,
// 4 fp32 channels in the generic one).
//
// Decode, same chapter, "single-token update maths", "the physical cache may exceed the
// minimal history", "state indices for continuous batching": one thread per (row, channel)
// reads its K-1 history values from the pool row into registers first, then produces the
// n_new outputs and only then writes the raw new inputs back into the ring (or shifts the
// linear row), so nothing it still needs is overwritten.
#include <type_traits>

#include "internal.h"

namespace ssm {
namespace {

constexpr int kConvThreads = 64;  // one wavefront per block
constexpr int kConvTokens = 32;   // tokens per thread run (>= K-1 for every K <= 8)

template <class D, int V>
struct Vec;
template <>
struct Vec<F32, 4> {
    __device__ static void load(const float* p, float (&v)[4]) {
        float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <class D>
struct Vec<D, 1> {
    __device__ static void load(const typename D::T* p, float (&v)[1]) { v[0] = D::load(p, 0); }
    __device__ static void store(typename D::T* p, const float (&v)[1]) { D::store(p, 0, v[0]); }
};

// Accumulation: fp32 for fp32 storage; double for bf16 storage, where the products of fp32
// weights and bf16 inputs are exact and the output's bf16 rounding then matches the exact
// conv value's (see act_to_bf16).
template <class D>
struct Acc;
template <>
struct Acc<F32> {
    using T = float;
    __device__ static float out(float z, int act) { return apply_act(z, act); }
};
template <>
struct Acc<BF16> {
    using T = double;
    // returns the bf16 result widened to float (exact), for the float-valued store path
    __device__ static float out(double z, int act) { return bf16_to_f32(act_to_bf16(z, act)); }
};

template <class D, int V, int K, bool HAS_SEQ>
__global__ void __launch_bounds__(kConvThreads)
conv1d_fwd_kernel(const typename D::T* __restrict__ x, const float* __restrict__ w,
                  const float* __restrict__ bias, const typename D::T* init_state,
                  typename D::T* final_state, const int32_t* __restrict__ seq_idx,
                  typename D::T* __restrict__ out, int64_t L, int64_t C, int act) {
    using T = typename D::T;
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x) * V;
    if (c0 >= C) return;
    const int64_t b = blockIdx.z;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kConvTokens;
    const int64_t t1 = min(t0 + kConvTokens, L);

    using AT = typename Acc<D>::T;
    AT wr[V][K];
    AT bv[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int k = 0; k < K; ++k) wr[v][k] = w[(c0 + v) * K + k];
        bv[v] = bias ? bias[c0 + v] : 0.0f;
    }

    // u-positions t0-K+1 .. t0-1 (oldest first): from x, or from the state for pos < 0
    AT hist[K - 1][V];
    int32_t hid[K - 1];
    const int32_t id0 = HAS_SEQ ? seq_idx[b * L] : 0;
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        const int64_t pos = t0 - (K - 1) + j;
        if (pos >= 0) {
            float tmp[V];
            Vec<D, V>::load(x + (b * L + pos) * C + c0, tmp);
#pragma unroll
            for (int v = 0; v < V; ++v) hist[j][v] = tmp[v];
            hid[j] = HAS_SEQ ? seq_idx[b * L + pos] : 0;
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v)
                hist[j][v] = init_state ? D::load(init_state, ((b * C + c0 + v) * (K - 1)) + (K - 1) + pos) : 0.0f;
            hid[j] = id0;
        }
    }

    for (int64_t t = t0; t < t1; ++t) {
        float xf[V];
        Vec<D, V>::load(x + (b * L + t) * C + c0, xf);
        const int32_t idt = HAS_SEQ ? seq_idx[b * L + t] : 0;
        float z[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const AT xv = xf[v];
            AT acc = bv[v];
#pragma unroll
            for (int k = 0; k < K - 1; ++k) {
                const AT tap = (!HAS_SEQ || hid[k] == idt) ? hist[k][v] : AT(0);
                acc = fma(wr[v][k], tap, acc);
            }
            acc = fma(wr[v][K - 1], xv, acc);
            z[v] = Acc<D>::out(acc, act);
        }
        Vec<D, V>::store(out + (b * L + t) * C + c0, z);
#pragma unroll
        for (int k = 0; k < K - 2; ++k) {
#pragma unroll
            for (int v = 0; v < V; ++v) hist[k][v] = hist[k + 1][v];
            hid[k] = hid[k + 1];
        }
#pragma unroll
        for (int v = 0; v < V; ++v) hist[K - 2][v] = xf[v];
        hid[K - 2] = idt;
    }

    // F = u[L .. L+K-2], written by the run that read the initial state (so an in-place
    // state pair is read before it is overwritten)
    if (final_state != nullptr && t0 == 0) {
        T fv[V][K - 1];
#pragma unroll
        for (int r = 0; r < K - 1; ++r) {
            const int64_t m = L + r;  // index into u
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if (m < K - 1) {
                    fv[v][r] = init_state ? init_state[(b * C + c0 + v) * (K - 1) + m] : T(0);
                } else {
                    fv[v][r] = x[(b * L + (m - (K - 1))) * C + c0 + v];
                }
            }
        }
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int r = 0; r < K - 1; ++r) final_state[(b * C + c0 + v) * (K - 1) + r] = fv[v][r];
    }
}

// bf16 prefill, the main case: each lane owns 2 adjacent channels of one batch row (4-byte
// loads and stores, 256 contiguous bytes per wavefront) and a run of kRun2 tokens.  Weights,
// bias and the K-1 previous inputs stay in registers as doubles.  Two channels keep a lane
// near 70 VGPRs, so seven wavefronts share a SIMD and one wave's loads overlap the others'
// arithmetic; four channels per lane needed 128 VGPRs (four waves) and ran 15-18% slower
// at the 1.3B layer shape, the same instructions per output either way.  The next group of
// kGroup2 tokens is loaded while the current group is computed.  SiLU outputs too close to
// a bf16 rounding midpoint for the fp32 evaluation (see silu_f32) are flagged (one mask per
// group, kept in the lane's own LDS words); after the run, when the fast path's registers
// are free, one loop recomputes the flagged outputs in double from memory and overwrites
// them.
constexpr int kRun2 = 32;   // tokens per lane run
constexpr int kGroup2 = 4;  // tokens per prefetch group
constexpr int kGroupsPerRun = kRun2 / kGroup2;

// Exact conv value at token t, channel ch of batch row b (the slow path's recomputation):
// taps at u-positions t-K+1 .. t, from x or from the initial state, each zeroed when its
// sequence id differs from token t's (positions before the row start carry token 0's id).
template <int K, bool HAS_SEQ>
__device__ double conv_exact_bf16(const uint16_t* x, const float* w, const float* bias,
                                  const uint16_t* init_state, const int32_t* srow, int64_t b,
                                  int64_t L, int64_t C, int64_t t, int64_t ch) {
    double z = bias ? bias[ch] : 0.0f;
    const int32_t idt = HAS_SEQ ? srow[t] : 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t pos = t - (K - 1) + k;
        double u;
        if (pos >= 0)
            u = bf16_to_f32(x[(b * L + pos) * C + ch]);
        else
            u = init_state ? bf16_to_f32(init_state[(b * C + ch) * (K - 1) + (K - 1) + pos]) : 0.0f;
        if (HAS_SEQ && srow[pos >= 0 ? pos : 0] != idt) u = 0.0;
        z = fma(static_cast<double>(w[ch * K + k]), u, z);
    }
    return z;
}

__device__ __forceinline__ void unpack2(uint32_t q, double (&v)[2]) {
    v[0] = __uint_as_float(q << 16);
    v[1] = __uint_as_float(q & 0xffff0000u);
}

template <int K, bool HAS_SEQ, bool SILU>
__global__ void __launch_bounds__(kConvThreads) __attribute__((amdgpu_waves_per_eu(4)))
conv1d_fwd_bf16x2_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                         const float* __restrict__ bias, const uint16_t* init_state,
                         uint16_t* final_state, const int32_t* __restrict__ seq_idx,
                         uint16_t* __restrict__ out, int64_t L, int64_t C) {
    constexpr int V = 2;
    const int64_t cblk = static_cast<int64_t>(blockIdx.x) * kConvThreads * V;
    const int64_t c0 = cblk + threadIdx.x * V;
    if (c0 >= C) return;
    const int64_t b = blockIdx.z;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kRun2;
    const int64_t t1 = min(t0 + kRun2, L);
    // a token row's base is uniform across the wavefront; each lane adds a 32-bit offset
    const uint16_t* xb = x + b * L * C + cblk;
    uint16_t* ob = out + b * L * C + cblk;
    const uint32_t lane_off = threadIdx.x * 4u;
    const int32_t* srow = HAS_SEQ ? seq_idx + b * L : nullptr;
    auto ld_hist = [&](int64_t t) {  // rows shared with the previous run: plain loads (L2)
        return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(xb + t * C) + lane_off);
    };
    auto ld_run = [&](int64_t t) {  // rows read once: non-temporal
        return __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(xb + t * C) + lane_off));
    };
    auto st_run = [&](int64_t t, uint32_t v) {
        __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ob + t * C) + lane_off));
    };

    // set-up loads carry no branches around them, so they are in flight together
    double wr[V][K], bv[V];
    const float* bsrc = bias ? bias : w;  // read either way; the value is dropped without bias
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int k = 0; k < K; ++k) wr[v][k] = w[(c0 + v) * K + k];
        const float bq = bsrc[c0 + v];
        bv[v] = bias ? bq : 0.0f;
    }
    // The window of a group: rows 0 .. K-2 hold the K-1 inputs before the group (oldest
    // first), row K-1+u the group's token u; output u takes rows u .. u+K-1.  First the
    // u-positions t0-K+1 .. t0-1: from x, or from the state for pos < 0.
    double win[kGroup2 + K - 1][V];
    int32_t wid[kGroup2 + K - 1];
    if (t0 >= K - 1) {
        uint32_t hq[K - 1];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            hq[j] = ld_hist(t0 - (K - 1) + j);
            wid[j] = HAS_SEQ ? srow[t0 - (K - 1) + j] : 0;
        }
#pragma unroll
        for (int j = 0; j < K - 1; ++j) unpack2(hq[j], win[j]);
    } else {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            const int64_t pos = t0 - (K - 1) + j;
            if (pos >= 0) {
                unpack2(ld_hist(pos), win[j]);
                wid[j] = HAS_SEQ ? srow[pos] : 0;
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v)
                    win[j][v] = init_state ? bf16_to_f32(init_state[(b * C + c0 + v) * (K - 1) + (K - 1) + pos]) : 0.0f;
                wid[j] = HAS_SEQ ? srow[0] : 0;
            }
        }
    }
    // a loaded group into window rows K-1 .. K+2
    auto fill = [&](const uint32_t (&xa)[kGroup2], const int32_t (&ia)[kGroup2]) {
#pragma unroll
        for (int u = 0; u < kGroup2; ++u) {
            unpack2(xa[u], win[K - 1 + u]);
            wid[K - 1 + u] = ia[u];
        }
    };
    // One group; FULL groups lie inside the run and skip the per-token bound checks; MASK
    // zeroes the taps from another sequence.  Bit 2*kGroup2-1 - (V*u + v) of the result flags
    // output (token tg+u, channel c0+v).
    auto group_body = [&](int64_t tg, auto full, auto mask) -> uint32_t {
        constexpr bool FULL = decltype(full)::value;
        constexpr bool MASK = decltype(mask)::value;
        uint32_t near = 0;
#pragma unroll
        for (int u = 0; u < kGroup2; ++u) {
            const int64_t t = tg + u;
            if (!FULL && t >= t1) {
                if (SILU) near <<= V;
                continue;
            }
            double z[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                double acc = bv[v];
#pragma unroll
                for (int k = 0; k < K - 1; ++k) {
                    const double tap = (!MASK || wid[u + k] == wid[u + K - 1]) ? win[u + k][v] : 0.0;
                    acc = fma(wr[v][k], tap, acc);
                }
                z[v] = fma(wr[v][K - 1], win[u + K - 1][v], acc);
            }
            uint16_t o[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if (SILU) {
                    bool nr;
                    o[v] = f32_to_bf16(silu_f32(z[v], nr));
                    near = near + near + static_cast<uint32_t>(nr);
                } else {
                    o[v] = f64_to_bf16(z[v]);
                }
            }
            st_run(t, o[0] | (static_cast<uint32_t>(o[1]) << 16));
        }
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
#pragma unroll
            for (int v = 0; v < V; ++v) win[j][v] = win[kGroup2 + j][v];
            wid[j] = wid[kGroup2 + j];
        }
        return near;
    };
    // sequence ids are wave-uniform: with SiLU, a window inside one sequence (the usual case)
    // takes the unmasked body, so only windows that cross a boundary pay for the per-tap
    // selects (the identity kernels and K = 8 keep one masked body: two bodies spill there)
    auto group = [&](int64_t tg, auto full) -> uint32_t {
        if constexpr (HAS_SEQ && SILU && K <= 7) {
            bool same = true;
#pragma unroll
            for (int j = 1; j < kGroup2 + K - 1; ++j) same = same && wid[j] == wid[0];
            if (!same) return group_body(tg, full, std::true_type{});
            return group_body(tg, full, std::false_type{});
        }
        return group_body(tg, full, std::bool_constant<HAS_SEQ>{});
    };
    static_assert(V * kGroup2 <= 32, "flag mask");
    __shared__ uint32_t flags[kGroupsPerRun][kConvThreads];
    if (t1 - t0 == kRun2) {
        // a whole run: every load in range, no per-token checks; the next group's loads are
        // issued before the current group's arithmetic and unpacked after it
        uint32_t xa[kGroup2];
        int32_t ia[kGroup2];
#pragma unroll
        for (int u = 0; u < kGroup2; ++u) {
            xa[u] = ld_run(t0 + u);
            ia[u] = HAS_SEQ ? srow[t0 + u] : 0;
        }
        fill(xa, ia);
#pragma unroll 1
        for (int g = 0; g < kGroupsPerRun - 1; ++g) {
#pragma unroll
            for (int u = 0; u < kGroup2; ++u) {
                xa[u] = ld_run(t0 + kGroup2 * (g + 1) + u);
                ia[u] = HAS_SEQ ? srow[t0 + kGroup2 * (g + 1) + u] : 0;
            }
            const uint32_t m = group(t0 + kGroup2 * g, std::true_type{});
            if (SILU) flags[g][threadIdx.x] = m;
            fill(xa, ia);
        }
        const uint32_t m = group(t0 + kGroup2 * (kGroupsPerRun - 1), std::true_type{});
        if (SILU) flags[kGroupsPerRun - 1][threadIdx.x] = m;
    } else {
        // the row's last, shorter run
        for (int64_t tg = t0; tg < t1; tg += kGroup2) {
            uint32_t xa[kGroup2];
            int32_t ia[kGroup2];
#pragma unroll
            for (int u = 0; u < kGroup2; ++u) {
                const int64_t t = tg + u;
                xa[u] = t < t1 ? ld_run(t) : 0u;
                ia[u] = HAS_SEQ && t < t1 ? srow[t] : 0;
            }
            fill(xa, ia);
            const uint32_t m = group(tg, std::false_type{});
            if (SILU) flags[(tg - t0) / kGroup2][threadIdx.x] = m;
        }
    }

    // rare: each iteration redoes one flagged output per lane (this lane stored the fast
    // value earlier, so the overwrite lands after it)
    if (SILU) {
        const int ng = static_cast<int>((t1 - t0 + kGroup2 - 1) / kGroup2);
        for (int g = 0; g < ng; ++g) {
            for (uint32_t m = flags[g][threadIdx.x]; m != 0; m &= m - 1) {
                const int idx = V * kGroup2 - 1 - __builtin_ctz(m);
                const int64_t t = t0 + g * kGroup2 + idx / V, ch = c0 + idx % V;
                const double z = conv_exact_bf16<K, HAS_SEQ>(x, w, bias, init_state, srow, b, L, C, t, ch);
                out[(b * L + t) * C + ch] = silu_f64_to_bf16(z);
            }
        }
    }

    // F = u[L .. L+K-2], written by the run that read the initial state (so an in-place
    // state pair is read before it is overwritten)
    if (final_state != nullptr && t0 == 0) {
        uint16_t fv[V][K - 1];
#pragma unroll
        for (int r = 0; r < K - 1; ++r) {
            const int64_t m = L + r;  // index into u
#pragma unroll
            for (int v = 0; v < V; ++v)
                fv[v][r] = m < K - 1 ? (init_state ? init_state[(b * C + c0 + v) * (K - 1) + m] : uint16_t(0))
                                     : x[(b * L + m - (K - 1)) * C + c0 + v];
        }
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int r = 0; r < K - 1; ++r) final_state[(b * C + c0 + v) * (K - 1) + r] = fv[v][r];
    }
}

template <int K>
hipError_t conv_fwd_bf16x2_dispatch_seq(const void* x, const float* w, const float* bias,
                                        const void* init_state, void* final_state,
                                        const int32_t* seq_idx, void* out, int64_t B, int64_t L,
                                        int64_t C, int act, hipStream_t stream) {
    const int64_t threads_needed = C / 2;
    dim3 grid((threads_needed + kConvThreads - 1) / kConvThreads,
              (L + kRun2 - 1) / kRun2, B);
    using U16 = uint16_t;
#define SSM_CONV2_LAUNCH(SEQ, SL)                                                             \
    conv1d_fwd_bf16x2_kernel<K, SEQ, SL><<<grid, kConvThreads, 0, stream>>>(                  \
        (const U16*)x, w, bias, (const U16*)init_state, (U16*)final_state, seq_idx, (U16*)out, \
        L, C)
    const bool silu = act == SSM_ACT_SILU;
    if (seq_idx) {
        if (silu) SSM_CONV2_LAUNCH(true, true);
        else SSM_CONV2_LAUNCH(true, false);
    } else {
        if (silu) SSM_CONV2_LAUNCH(false, true);
        else SSM_CONV2_LAUNCH(false, false);
    }
#undef SSM_CONV2_LAUNCH
    return hipGetLastError();
}

hipError_t conv_fwd_bf16x2_dispatch(int64_t K, const void* x, const float* w, const float* bias,
                                    const void* init_state, void* final_state,
                                    const int32_t* seq_idx, void* out, int64_t B, int64_t L,
                                    int64_t C, int act, hipStream_t stream) {
#define SSM_CONV2_K(KK)                                                                      \
    case KK:                                                                                 \
        return conv_fwd_bf16x2_dispatch_seq<KK>(x, w, bias, init_state, final_state, seq_idx, \
                                                out, B, L, C, act, stream);
    switch (K) {
        SSM_CONV2_K(2) SSM_CONV2_K(3) SSM_CONV2_K(4) SSM_CONV2_K(5) SSM_CONV2_K(6)
        SSM_CONV2_K(7) SSM_CONV2_K(8)
        default: return hipErrorInvalidValue;
    }
#undef SSM_CONV2_K
}

// seqlen == 0: F = S (or zeros)
template <class D>
__global__ void conv_state_passthrough_kernel(const typename D::T* init_state,
                                              typename D::T* final_state, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) final_state[i] = init_state ? init_state[i] : typename D::T(0);
}

template <class D, int V, int K>
hipError_t conv_fwd_dispatch_seq(const void* x, const float* w, const float* bias,
                                 const void* init_state, void* final_state,
                                 const int32_t* seq_idx, void* out, int64_t B, int64_t L,
                                 int64_t C, int act, hipStream_t stream) {
    using T = typename D::T;
    const int64_t threads_needed = (C + V - 1) / V;
    dim3 grid((threads_needed + kConvThreads - 1) / kConvThreads,
              (L + kConvTokens - 1) / kConvTokens, B);
    if (seq_idx)
        conv1d_fwd_kernel<D, V, K, true><<<grid, kConvThreads, 0, stream>>>(
            (const T*)x, w, bias, (const T*)init_state, (T*)final_state, seq_idx, (T*)out, L,
            C, act);
    else
        conv1d_fwd_kernel<D, V, K, false><<<grid, kConvThreads, 0, stream>>>(
            (const T*)x, w, bias, (const T*)init_state, (T*)final_state, seq_idx, (T*)out, L,
            C, act);
    return hipGetLastError();
}

template <class D, int V>
hipError_t conv_fwd_dispatch_k(int64_t K, const void* x, const float* w, const float* bias,
                               const void* init_state, void* final_state,
                               const int32_t* seq_idx, void* out, int64_t B, int64_t L,
                               int64_t C, int act, hipStream_t stream) {
#define SSM_CONV_K(KK)                                                                    \
    case KK:                                                                              \
        return conv_fwd_dispatch_seq<D, V, KK>(x, w, bias, init_state, final_state,      \
                                               seq_idx, out, B, L, C, act, stream);
    switch (K) {
        SSM_CONV_K(2) SSM_CONV_K(3) SSM_CONV_K(4) SSM_CONV_K(5) SSM_CONV_K(6) SSM_CONV_K(7)
        SSM_CONV_K(8)
        default: return hipErrorInvalidValue;
    }
#undef SSM_CONV_K
}

// ---------------------------------------------------------------------------------------
// decode update
// ---------------------------------------------------------------------------------------
template <class D, int K>
__global__ void __launch_bounds__(256)
conv1d_update_kernel(const typename D::T* __restrict__ x, typename D::T* pool,
                     const float* __restrict__ w, const float* __restrict__ bias,
                     const int32_t* __restrict__ indices, const int32_t* __restrict__ seqlens,
                     typename D::T* __restrict__ out, int64_t C, int64_t L_new,
                     int64_t state_len, int64_t n_slots, int act) {
    using T = typename D::T;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (c >= C) return;
    const int64_t b = blockIdx.y;
    const int64_t s = indices ? static_cast<int64_t>(indices[b]) : b;
    T* o = out + (b * C + c) * L_new;
    if (s < 0 || s >= n_slots) {
        for (int64_t i = 0; i < L_new; ++i) D::store(o, i, 0.0f);
        return;
    }
    T* row = pool + (s * C + c) * state_len;
    const T* xr = x + (b * C + c) * L_new;
    const int64_t p = seqlens ? static_cast<int64_t>(seqlens[b]) : 0;

    using AT = typename Acc<D>::T;
    AT wr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wr[k] = w[c * K + k];
    const AT bv = bias ? bias[c] : 0.0f;

    if constexpr (std::is_same<D, BF16>::value && K <= 5) {
        // bf16 rows of 4 entries (the usual width-4 decode cache): the row is one 8-byte word,
        // read once, updated in a register (ring insert, or shift for the linear layout) and
        // written once; entry k sits in bits 16k .. 16k + 15.  Same arithmetic as below.
        if (state_len == 4 && (reinterpret_cast<uintptr_t>(row) & 7) == 0) {
            uint64_t r64 = *reinterpret_cast<const uint64_t*>(row);
            auto entry = [&](int64_t slot) -> AT {
                return bf16_to_f32(static_cast<uint16_t>(r64 >> (16 * slot)));
            };
            AT hist4[K - 1];
#pragma unroll
            for (int j = 1; j <= K - 1; ++j)
                hist4[K - 1 - j] = entry(seqlens ? floor_mod(p - j, 4) : 4 - j);
            for (int64_t i = 0; i < L_new; ++i) {
                const uint16_t xb = xr[i];
                const AT xv = bf16_to_f32(xb);
                AT acc = bv;
#pragma unroll
                for (int k = 0; k < K - 1; ++k) acc = fma(wr[k], hist4[k], acc);
                acc = fma(wr[K - 1], xv, acc);
                D::store(o, i, Acc<D>::out(acc, act));
#pragma unroll
                for (int k = 0; k < K - 2; ++k) hist4[k] = hist4[k + 1];
                hist4[K - 2] = xv;
                if (seqlens) {
                    const int sh = 16 * static_cast<int>(floor_mod(p + i, 4));
                    r64 = (r64 & ~(0xFFFFull << sh)) | (static_cast<uint64_t>(xb) << sh);
                } else {
                    r64 = (r64 >> 16) | (static_cast<uint64_t>(xb) << 48);
                }
            }
            *reinterpret_cast<uint64_t*>(row) = r64;
            return;
        }
    }

    // history, oldest first: hist[K-1-j] = value j steps back (read before any write)
    AT hist[K - 1];
#pragma unroll
    for (int j = 1; j <= K - 1; ++j) {
        const int64_t slot = seqlens ? floor_mod(p - j, state_len) : state_len - j;
        hist[K - 1 - j] = D::load(row, slot);
    }
    for (int64_t i = 0; i < L_new; ++i) {
        const AT xv = D::load(xr, i);
        AT acc = bv;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) acc = fma(wr[k], hist[k], acc);
        acc = fma(wr[K - 1], xv, acc);
        D::store(o, i, Acc<D>::out(acc, act));
#pragma unroll
        for (int k = 0; k < K - 2; ++k) hist[k] = hist[k + 1];
        hist[K - 2] = xv;
    }
    // write the raw inputs (never the outputs) back into the cache
    if (seqlens) {
        for (int64_t i = 0; i < L_new; ++i) row[floor_mod(p + i, state_len)] = xr[i];
    } else {
        // row <- last state_len entries of (row ++ x); sources sit at or after their
        // destinations, so a forward copy is safe in place
        for (int64_t i = 0; i < state_len; ++i) {
            const int64_t q = L_new + i;
            row[i] = q < state_len ? row[q] : xr[q - state_len];
        }
    }
}

template <class D>
hipError_t conv_update_dispatch(int64_t K, const void* x, void* pool, const float* w,
                                const float* bias, const int32_t* indices,
                                const int32_t* seqlens, void* out, int64_t B, int64_t C,
                                int64_t L_new, int64_t state_len, int64_t n_slots, int act,
                                hipStream_t stream) {
    using T = typename D::T;
    dim3 grid((C + 255) / 256, B);
#define SSM_UPD_K(KK)                                                                      \
    case KK:                                                                               \
        conv1d_update_kernel<D, KK><<<grid, 256, 0, stream>>>(                             \
            (const T*)x, (T*)pool, w, bias, indices, seqlens, (T*)out, C, L_new, state_len, \
            n_slots, act);                                                                 \
        break;
    switch (K) {
        SSM_UPD_K(2) SSM_UPD_K(3) SSM_UPD_K(4) SSM_UPD_K(5) SSM_UPD_K(6) SSM_UPD_K(7)
        SSM_UPD_K(8)
        default: return hipErrorInvalidValue;
    }
#undef SSM_UPD_K
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d_fwd(const void* x, const float* w, const float* bias,
                             const void* init_state, void* final_state, const int32_t* seq_idx,
                             void* out, int64_t B, int64_t L, int64_t C, int64_t K,
                             ssm_dtype_t dtype, int act, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    if (L == 0) {
        if (!final_state) return hipSuccess;
        const int64_t n = B * C * (K - 1);
        const int blocks = static_cast<int>((n + 255) / 256);
        if (dtype == SSM_BF16)
            conv_state_passthrough_kernel<BF16><<<blocks, 256, 0, stream>>>(
                (const uint16_t*)init_state, (uint16_t*)final_state, n);
        else
            conv_state_passthrough_kernel<F32><<<blocks, 256, 0, stream>>>(
                (const float*)init_state, (float*)final_state, n);
        return hipGetLastError();
    }
    const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out);
    if (dtype == SSM_BF16) {
        if (C % 2 == 0 && (align & 3) == 0)
            return conv_fwd_bf16x2_dispatch(K, x, w, bias, init_state, final_state, seq_idx, out,
                                            B, L, C, act, stream);
        return conv_fwd_dispatch_k<BF16, 1>(K, x, w, bias, init_state, final_state, seq_idx,
                                           out, B, L, C, act, stream);
    }
    if (C % 4 == 0 && (align & 15) == 0)
        return conv_fwd_dispatch_k<F32, 4>(K, x, w, bias, init_state, final_state, seq_idx, out,
                                          B, L, C, act, stream);
    return conv_fwd_dispatch_k<F32, 1>(K, x, w, bias, init_state, final_state, seq_idx, out, B,
                                      L, C, act, stream);
}

hipError_t launch_conv1d_update(const void* x, void* pool, const float* w, const float* bias,
                                const int32_t* indices, const int32_t* cache_seqlens, void* out,
                                int64_t B, int64_t C, int64_t L_new, int64_t K,
                                int64_t state_len, int64_t n_slots, ssm_dtype_t dtype, int act,
                                hipStream_t stream) {
    if (B == 0 || L_new == 0) return hipSuccess;
    if (dtype == SSM_BF16)
        return conv_update_dispatch<BF16>(K, x, pool, w, bias, indices, cache_seqlens, out, B, C,
                                          L_new, state_len, n_slots, act, stream);
    return conv_update_dispatch<F32>(K, x, pool, w, bias, indices, cache_seqlens, out, B, C,
                                     L_new, state_len, n_slots, act, stream);
}

}  // namespace ssm
