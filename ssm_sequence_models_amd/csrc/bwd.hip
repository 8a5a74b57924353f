// bwd.hip -- backward kernels with state gradients.
//
// conv1d backward (causal-conv1d tutorial, ch. 7, "backward with states, a unified
// derivation" and "chunked training and truncated back-propagation"): over the extended
// sequence u = [S, x] and with delta_t = dL/dz_t = dy_t phi'(z_t),
//     du_j = sum_t sum_k delta_t w_k [j = t + k] + [L <= j < L+K-1] q_{j-L},
//     dS = du[0 : K-1],  dx = du[K-1 : K-1+L],  dw_k = sum delta_t u_{t+k},  dbeta = sum delta_t,
// with the forward's sequence masks on the taps (q = dL/dF reaches the last K-1 inputs
// directly, unmasked, as F is their raw copy).
//
// Initial-state gradient of the scan (length-generalization reading notes, Sec. 2.5 Eq. (4)
// and Sec. 2.6): h_{-1} reaches y_t through C_t^T (prod_{tau<=t} a_tau) h_{-1}, so
//     dh_{-1}[p][n] = sum_t dy_t[p] E_t C_t[n] + E_{L-1} dF[p][n],   E_t = prod_{tau<=t} a_tau,
// where a packed-sequence change cuts h_{-1} off from every later token (and from F).
#include "internal.h"

namespace ssm {
namespace {

// ---------------------------------------------------------------------------------------
// conv1d backward: thread = (row b, channel c, run r of kConvBwdRun tokens).  The thread
// walks tokens t0 .. t1+K-2: it recomputes z_t from a register window of the K inputs of
// output t, forms delta_t, adds the run's own tokens to its dw / dbeta partial sums, and
// emits dx_s for s = t-K+1 once delta_{s .. s+K-1} are known.  Run 0 also forms dS from
// delta_0 .. delta_{K-2}.  Consecutive threads take consecutive channels (coalesced rows).
// Used for fp32, odd channel counts and unaligned rows; bf16 rows of whole 2-channel groups
// take conv1d_bwd_bf16vec_kernel below.
// ---------------------------------------------------------------------------------------
constexpr int kConvBwdRun = 64;
constexpr int kConvBwdThreads = 256;
constexpr int kBwdGroup = 4;  // tokens per group of the bf16 vector kernel's main range

template <class D, int K>
__global__ void __launch_bounds__(kConvBwdThreads)
conv1d_bwd_kernel(const typename D::T* x, const float* w, const float* bias,
                  const typename D::T* init, const int32_t* seq, const typename D::T* dy,
                  const typename D::T* dfin, typename D::T* dx, typename D::T* dinit,
                  float* part, int64_t L, int64_t C, int nruns, int silu) {
    using T = typename D::T;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * kConvBwdThreads + threadIdx.x;
    const int r = blockIdx.y;
    const int64_t b = blockIdx.z;
    if (c >= C) return;  // no barriers in this kernel
    const int64_t t0 = static_cast<int64_t>(r) * kConvBwdRun;
    const int64_t t1 = min(t0 + kConvBwdRun, L);
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = w[c * K + k];
    const float beta = bias ? bias[c] : 0.0f;
    const int32_t* sq = seq ? seq + b * L : nullptr;
    const int32_t id0 = sq ? sq[0] : 0;
    // input at x index s (s < 0: the state, S_{K-1+s}) and its token identity
    auto xval = [&](int64_t s) -> float {
        if (s >= 0) return D::load(x, (b * L + s) * C + c);
        return init ? D::load(init, (b * C + c) * (K - 1) + (K - 1) + s) : 0.0f;
    };
    auto sid = [&](int64_t s) -> int32_t { return sq ? sq[s < 0 ? 0 : s] : 0; };

    float xv[K];     // inputs of output t: x indices t-K+1 .. t
    int32_t xs[K];   // their identities
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        xv[k + 1] = xval(t0 - (K - 1) + k);
        xs[k + 1] = sid(t0 - (K - 1) + k);
    }
    float dl[K];     // delta of tokens t-K+1 .. t (0 past the row's end)
    int32_t ds[K];   // identities of those tokens
#pragma unroll
    for (int k = 0; k < K; ++k) {
        dl[k] = 0.0f;
        ds[k] = 0;
    }
    float dwp[K], dbp = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) dwp[k] = 0.0f;
    float dsd[K];    // delta_0 .. delta_{K-2} (run 0: the dS terms)
    int32_t dss[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        dsd[k] = 0.0f;
        dss[k] = id0;
    }

    for (int64_t t = t0; t < t1 + K - 1; ++t) {
        const bool live = t < L;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            xv[k] = xv[k + 1];
            xs[k] = xs[k + 1];
            dl[k] = dl[k + 1];
            ds[k] = ds[k + 1];
        }
        float delta = 0.0f;
        int32_t idt = 0;
        if (live) {
            xv[K - 1] = D::load(x, (b * L + t) * C + c);
            xs[K - 1] = idt = sid(t);
            float z = beta;
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (!sq || xs[k] == idt) z = __builtin_fmaf(wk[k], xv[k], z);
            float dphi = 1.0f;
            if (silu) {
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
                dphi = sg * (1.0f + z * (1.0f - sg));
            }
            delta = D::load(dy, (b * L + t) * C + c) * dphi;
            if (t < t1) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (!sq || xs[k] == idt) dwp[k] = __builtin_fmaf(delta, xv[k], dwp[k]);
                dbp += delta;
            }
            if (t < K - 1) {
#pragma unroll
                for (int k = 0; k < K - 1; ++k)
                    if (k == t) {
                        dsd[k] = delta;
                        dss[k] = idt;
                    }
            }
        }
        dl[K - 1] = delta;
        ds[K - 1] = idt;
        // dx_s, s = t-K+1: taps m = 0 .. K-1 of outputs s+m through weight K-1-m
        const int64_t s = t - (K - 1);
        if (s >= t0 && s < t1) {
            const int32_t ids = ds[0];  // identity of token s (its own output, m = 0)
            float v = 0.0f;
#pragma unroll
            for (int m = 0; m < K; ++m)
                if (!sq || ds[m] == ids) v = __builtin_fmaf(dl[m], wk[K - 1 - m], v);
            if (dfin && s + K - 1 >= L) v += D::load(dfin, (b * C + c) * (K - 1) + (s + K - 1 - L));
            D::store(dx, (b * L + s) * C + c, v);
        }
    }
    if (r == 0 && dinit) {
        // dS_j = sum_{t <= j} delta_t w_{j-t} (taps whose identity, the state's, matches
        // output t) + q_{j-L} when j >= L
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            float v = 0.0f;
#pragma unroll
            for (int t = 0; t <= j; ++t)
                if (t < L && (!sq || dss[t] == id0)) v = __builtin_fmaf(dsd[t], wk[j - t], v);
            if (dfin && j >= L) v += D::load(dfin, (b * C + c) * (K - 1) + (j - L));
            D::store(dinit, (b * C + c) * (K - 1) + j, v);
        }
    }
    float* pp = part + ((b * nruns + r) * C + c) * (K + 1);
#pragma unroll
    for (int k = 0; k < K; ++k) pp[k] = dwp[k];
    pp[K] = dbp;
}

// The same walk for bf16 with V adjacent channels per thread (C % V == 0, x / dy / dx
// aligned to 2V bytes): each load and store of x, dy and dx moves 2V bytes, and the token
// identities and the sequence masks are shared by the V channels.  V = 2 is the one
// launched: about 70 VGPRs, so seven wavefronts share a SIMD and one wave's loads overlap the
// others' arithmetic, where V = 4 needed 118 VGPRs (four waves).
template <int V>
struct BwdVec;
template <>
struct BwdVec<4> {
    using Q = uint2;
    __device__ static Q ld(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ static Q ld_stream(const uint16_t* p) { return ld_stream_u2(p); }
    __device__ static void st_stream(uint16_t* p, const float (&v)[4]) {
        st_stream_u2(p, uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    }
    __device__ static void unpack(Q r, float (&v)[4]) {
        v[0] = __uint_as_float(r.x << 16);
        v[1] = __uint_as_float(r.x & 0xFFFF0000u);
        v[2] = __uint_as_float(r.y << 16);
        v[3] = __uint_as_float(r.y & 0xFFFF0000u);
    }
};
template <>
struct BwdVec<2> {
    using Q = uint32_t;
    __device__ static Q ld(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
    __device__ static Q ld_stream(const uint16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    __device__ static void st_stream(uint16_t* p, const float (&v)[2]) {
        __builtin_nontemporal_store(pack_bf16x2(v[0], v[1]), reinterpret_cast<uint32_t*>(p));
    }
    __device__ static void unpack(Q r, float (&v)[2]) {
        v[0] = __uint_as_float(r << 16);
        v[1] = __uint_as_float(r & 0xFFFF0000u);
    }
};

template <int K, int V>
__global__ void __launch_bounds__(kConvBwdThreads)
conv1d_bwd_bf16vec_kernel(const uint16_t* x, const float* w, const float* bias,
                          const uint16_t* init, const int32_t* seq, const uint16_t* dy,
                          const uint16_t* dfin, uint16_t* dx, uint16_t* dinit, float* part,
                          int64_t L, int64_t C, int nruns, int silu) {
    using VQ = BwdVec<V>;
    using Q = typename VQ::Q;
    // block = 64 groups of V channels x four consecutive runs, one run per wavefront; the four runs'
    // dw / dbeta partial sums are added in the block (in order) before they leave
    // the wave index through readfirstlane: the compiler then keeps the run's token bounds in
    // scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t cv = (static_cast<int64_t>(blockIdx.x) * 64 + lane) * V;
    const int r = 4 * static_cast<int>(blockIdx.y) + wave;
    const int64_t b = blockIdx.z;
    float dwp[K][V], dbp[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        dbp[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) dwp[k][j] = 0.0f;
    }
    if (cv < C && r < nruns) {
    const int64_t t0 = static_cast<int64_t>(r) * kConvBwdRun;
    const int64_t t1 = min(t0 + kConvBwdRun, L);
    // The set-up loads carry no branches around them, so they are in flight together: the
    // weights, the bias (read from w when there is none, and dropped), the x and dy of the
    // run's first K-1 tokens (clamped into the row) and the K-1 inputs before the run.
    float wk[K][V], beta[V];
    const float* bsrc = bias ? bias : w;
#pragma unroll
    for (int j = 0; j < V; ++j) {
#pragma unroll
        for (int k = 0; k < K; ++k) wk[k][j] = w[(cv + j) * K + k];
        const float bq = bsrc[cv + j];
        beta[j] = bias ? bq : 0.0f;
    }
    const int32_t* sq = seq ? seq + b * L : nullptr;
    const int32_t id0 = sq ? sq[0] : 0;
    auto sid = [&](int64_t s) -> int32_t { return sq ? sq[s < 0 ? 0 : s] : 0; };
    auto load4 = [&](const uint16_t* p, int64_t t, float (&v)[V]) {
        VQ::unpack(VQ::ld(p + (b * L + t) * C + cv), v);
    };
    Q hx[K - 1], hg[K - 1];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        const int64_t tc = min(t0 + k, L - 1);
        hx[k] = VQ::ld(x + (b * L + tc) * C + cv);
        hg[k] = VQ::ld(dy + (b * L + tc) * C + cv);
    }

    float xv[K][V];   // inputs of output t: x indices t-K+1 .. t
    int32_t xs[K];    // their identities
    if (t0 >= K - 1) {
        Q hq[K - 1];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) hq[k] = VQ::ld(x + (b * L + t0 - (K - 1) + k) * C + cv);
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            VQ::unpack(hq[k], xv[k + 1]);
            xs[k + 1] = sid(t0 - (K - 1) + k);
        }
    } else {
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            const int64_t s_ = t0 - (K - 1) + k;
            if (s_ >= 0) {
                load4(x, s_, xv[k + 1]);
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    xv[k + 1][j] = init ? bf16_to_f32(init[(b * C + cv + j) * (K - 1) + (K - 1) + s_]) : 0.0f;
            }
            xs[k + 1] = sid(s_);
        }
    }
    float dl[K][V];   // delta of tokens t-K+1 .. t (0 past the row's end)
    int32_t ds[K];
    float dsd[K][V];
    int32_t dss[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        ds[k] = 0;
        dss[k] = id0;
#pragma unroll
        for (int j = 0; j < V; ++j) dl[k][j] = dsd[k][j] = 0.0f;
    }

    // one token, general case (the run's first K-1 tokens, its last K-1 steps and short
    // runs); PRE: x_t and dy_t already loaded (qx, qg), else loaded here
    auto token = [&](int64_t t, Q qx, Q qg, auto pre) {
        constexpr bool PRE = decltype(pre)::value;
        const bool live = t < L;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            xs[k] = xs[k + 1];
            ds[k] = ds[k + 1];
#pragma unroll
            for (int j = 0; j < V; ++j) {
                xv[k][j] = xv[k + 1][j];
                dl[k][j] = dl[k + 1][j];
            }
        }
        float delta[V] = {};
        int32_t idt = 0;
        if (live) {
            float g[V];
            if (PRE) {
                VQ::unpack(qx, xv[K - 1]);
                VQ::unpack(qg, g);
            } else {
                load4(x, t, xv[K - 1]);
                load4(dy, t, g);
            }
            xs[K - 1] = idt = sid(t);
            bool tap[K];
#pragma unroll
            for (int k = 0; k < K; ++k) tap[k] = !sq || xs[k] == idt;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                float z = beta[j];
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (tap[k]) z = __builtin_fmaf(wk[k][j], xv[k][j], z);
                float dphi = 1.0f;
                if (silu) {
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
                    dphi = sg * (1.0f + z * (1.0f - sg));
                }
                delta[j] = g[j] * dphi;
            }
            if (t < t1) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (tap[k]) {
#pragma unroll
                        for (int j = 0; j < V; ++j) dwp[k][j] = __builtin_fmaf(delta[j], xv[k][j], dwp[k][j]);
                    }
#pragma unroll
                for (int j = 0; j < V; ++j) dbp[j] += delta[j];
            }
            if (t < K - 1) {
#pragma unroll
                for (int k = 0; k < K - 1; ++k)
                    if (k == t) {
                        dss[k] = idt;
#pragma unroll
                        for (int j = 0; j < V; ++j) dsd[k][j] = delta[j];
                    }
            }
        }
#pragma unroll
        for (int j = 0; j < V; ++j) dl[K - 1][j] = delta[j];
        ds[K - 1] = idt;
        // dx_s, s = t-K+1: taps m = 0 .. K-1 of outputs s+m through weight K-1-m
        const int64_t s_ = t - (K - 1);
        if (s_ >= t0 && s_ < t1) {
            const int32_t ids = ds[0];
            float v[V] = {};
#pragma unroll
            for (int m = 0; m < K; ++m)
                if (!sq || ds[m] == ids) {
#pragma unroll
                    for (int j = 0; j < V; ++j) v[j] = __builtin_fmaf(dl[m][j], wk[K - 1 - m][j], v[j]);
                }
            if (dfin && s_ + K - 1 >= L) {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    v[j] += bf16_to_f32(dfin[(b * C + cv + j) * (K - 1) + (s_ + K - 1 - L)]);
            }
            VQ::st_stream(dx + (b * L + s_) * C + cv, v);
        }
    };
    // Tokens ta .. tb-1 (all inside the run, at least K-1 after its start) in groups of
    // kBwdGroup: every token is live, accumulates into dw / dbeta and emits dx for s = t-K+1
    // inside the run, so no per-token checks.  The inputs, deltas and identities sit in
    // windows (rows 0 .. K-2 the K-1 before the group, row K-1+u token u) that move once per
    // group, and the next group's x and dy load while this one is computed.  Same arithmetic
    // in the same order as the general case.
    const int64_t ta = min(t0 + K - 1, t1), tb = t1;
    int64_t t = t0;
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
        if (t < ta) {
            token(t, hx[k], hg[k], std::true_type{});
            ++t;
        }
    if (tb - t >= kBwdGroup) {
        constexpr int G = kBwdGroup;
        float xw[G + K - 1][V], dlw[G + K - 1][V];
        int32_t idw[G + K - 1];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                xw[j][v] = xv[j + 1][v];
                dlw[j][v] = dl[j + 1][v];
            }
            idw[j] = xs[j + 1];
        }
        Q xq[G], gq[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            xq[u] = VQ::ld_stream(x + (b * L + t + u) * C + cv);
            gq[u] = VQ::ld_stream(dy + (b * L + t + u) * C + cv);
        }
        for (; t + G <= tb; t += G) {
            Q xn[G], gn[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int64_t tt = t + G + u;
                xn[u] = tt < L ? VQ::ld_stream(x + (b * L + tt) * C + cv) : Q{};
                gn[u] = tt < L ? VQ::ld_stream(dy + (b * L + tt) * C + cv) : Q{};
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                VQ::unpack(xq[u], xw[K - 1 + u]);
                idw[K - 1 + u] = sid(t + u);
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                float g[V];
                VQ::unpack(gq[u], g);
                bool tap[K];
#pragma unroll
                for (int k = 0; k < K; ++k) tap[k] = !sq || idw[u + k] == idw[u + K - 1];
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    float z = beta[j];
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        if (tap[k]) z = __builtin_fmaf(wk[k][j], xw[u + k][j], z);
                    float dphi = 1.0f;
                    if (silu) {
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
                        dphi = sg * (1.0f + z * (1.0f - sg));
                    }
                    dlw[K - 1 + u][j] = g[j] * dphi;
                }
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (tap[k]) {
#pragma unroll
                        for (int j = 0; j < V; ++j) dwp[k][j] = __builtin_fmaf(dlw[K - 1 + u][j], xw[u + k][j], dwp[k][j]);
                    }
#pragma unroll
                for (int j = 0; j < V; ++j) dbp[j] += dlw[K - 1 + u][j];
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int64_t s_ = t + u - (K - 1);
                float v[V] = {};
#pragma unroll
                for (int m = 0; m < K; ++m)
                    if (!sq || idw[u + m] == idw[u]) {
#pragma unroll
                        for (int j = 0; j < V; ++j) v[j] = __builtin_fmaf(dlw[u + m][j], wk[K - 1 - m][j], v[j]);
                    }
                VQ::st_stream(dx + (b * L + s_) * C + cv, v);
            }
#pragma unroll
            for (int j = 0; j < K - 1; ++j) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    xw[j][v] = xw[G + j][v];
                    dlw[j][v] = dlw[G + j][v];
                }
                idw[j] = idw[G + j];
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                xq[u] = xn[u];
                gq[u] = gn[u];
            }
        }
        // back to the general case's windows (inputs and deltas of the last K-1 tokens)
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                xv[j + 1][v] = xw[j][v];
                dl[j + 1][v] = dlw[j][v];
            }
            xs[j + 1] = ds[j + 1] = idw[j];
        }
        // the loop's last prefetch holds x and dy of the next G tokens (zeros past the row)
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (t < t1 + K - 1) {
                token(t, xq[u], gq[u], std::true_type{});
                ++t;
            }
    }
    for (; t < t1 + K - 1; ++t) token(t, Q{}, Q{}, std::false_type{});
    if (r == 0 && dinit) {
#pragma unroll
        for (int jj = 0; jj < K - 1; ++jj) {
#pragma unroll
            for (int j = 0; j < V; ++j) {
                float v = 0.0f;
#pragma unroll
                for (int t = 0; t <= jj; ++t)
                    if (t < L && (!sq || dss[t] == id0)) v = __builtin_fmaf(dsd[t][j], wk[jj - t][j], v);
                if (dfin && jj >= L) v += bf16_to_f32(dfin[(b * C + cv + j) * (K - 1) + (jj - L)]);
                dinit[(b * C + cv + j) * (K - 1) + jj] = f32_to_bf16(v);
            }
        }
    }
    }
    __shared__ float red[4][K + 1][V][64];
#pragma unroll
    for (int j = 0; j < V; ++j) {
#pragma unroll
        for (int k = 0; k < K; ++k) red[wave][k][j][lane] = dwp[k][j];
        red[wave][K][j][lane] = dbp[j];
    }
    __syncthreads();
    if (wave == 0 && cv < C) {
        const int64_t ngroups = (nruns + 3) / 4;
        float* pp = part + ((b * ngroups + blockIdx.y) * C + cv) * (K + 1);
#pragma unroll
        for (int j = 0; j < V; ++j)
#pragma unroll
            for (int k = 0; k <= K; ++k) {
                const double v = ((static_cast<double>(red[0][k][j][lane]) + red[1][k][j][lane]) +
                                  red[2][k][j][lane]) + red[3][k][j][lane];
                pp[j * (K + 1) + k] = static_cast<float>(v);
            }
    }
}

// dw[c][k] and dbias[c]: the runs' partial sums added in a fixed order, in double.  A block
// takes 64 consecutive outputs (one per lane); its four wavefronts sum a quarter of the
// partials each, and wave 0 adds the four in order.
__global__ void __launch_bounds__(256)
conv1d_bwd_reduce_kernel(const float* part, float* dw, float* dbias, int64_t C, int K,
                         int64_t nparts) {
    __shared__ double red[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t n = C * (K + 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    double acc = 0.0;
    if (i < n) {
        const int64_t p0 = wv * nparts / 4, p1 = (wv + 1) * nparts / 4;
#pragma unroll 8
        for (int64_t p = p0; p < p1; ++p) acc += part[p * n + i];
    }
    red[wv][lane] = acc;
    __syncthreads();
    if (wv == 0 && i < n) {
        const double v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        const int64_t c = i / (K + 1), k = i % (K + 1);
        if (k < K) dw[c * K + k] = static_cast<float>(v);
        else if (dbias) dbias[c] = static_cast<float>(v);
    }
}

__global__ void fill_zero_f32_kernel(float* p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// L = 0: dS = q (F is S itself), dw = dbias = 0
template <class D>
__global__ void conv1d_bwd_empty_kernel(const typename D::T* dfin, typename D::T* dinit, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n && dinit) D::store(dinit, i, dfin ? D::load(dfin, i) : 0.0f);
}

// ---------------------------------------------------------------------------------------
// dh_{-1}, MFMA path (P = 64, N = 128, bf16): one block per (b, h, column half), four
// wavefronts; wave w owns rows p = 16 w .. 16 w + 15 of the half in accumulators.  Per chunk:
// dy^T and C^T are staged in LDS (token index contiguous), wave 0 forms E_t = 2^(offset +
// prefix of dt A log2 e) with a DPP scan, then dh += (E o dy)^T C with E o dy split into two
// bf16 halves (hi + lo, as the main scan) against the exact bf16 C.  The loop stops at the
// first packed-sequence change and once E underflows to 0: every later term is exactly 0.
// ---------------------------------------------------------------------------------------
constexpr int kH0Q = 64, kH0P = 64, kH0N = 128;
constexpr int kH0Row = kH0Q * 2 + 16;  // bytes per [row][64 tokens] bf16 row in LDS (padded)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float h0_incl_sum(float v) {
    const int z = __float_as_int(0.0f);
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x118, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}

// Block = (b, h, half of the 128 state columns), so two blocks share a CU.  Per 64-token
// chunk each thread moves one 16-byte piece of two consecutive token rows of C and of dy into
// LDS transposed ([column][token]), packing the two tokens into one 4-byte store (consecutive
// lanes take consecutive token pairs: conflict-free stores).  The loads for chunk k+1 are
// issued before chunk k's products and stored after them, into the other of two buffers.
__global__ void __launch_bounds__(256)
scan_bwd_h0_mfma_kernel(const float* dt, const float* A, const uint16_t* Cm,
                        const int32_t* seq, const uint16_t* dy, const float* dfin, float* dh0,
                        int64_t L, int64_t H, int64_t G) {
    constexpr int kNh = kH0N / 2;  // columns per block
    __shared__ __attribute__((aligned(16))) uint8_t sCt[2][kNh * kH0Row];  // C^T [n][t]
    __shared__ __attribute__((aligned(16))) uint8_t sDy[2][kH0P * kH0Row];  // dy^T [p][t]
    __shared__ float sE[2][kH0Q];
    __shared__ int sStop[2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, g4 = lane >> 4;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int nh = blockIdx.z;
    const int64_t g = h / (H / G);
    const float a2 = A[h] * 1.4426950408889634f;
    const int32_t* sq = seq ? seq + b * L : nullptr;
    const int64_t nchunks = (L + kH0Q - 1) / kH0Q;
    // this thread's staging unit: token pair tp, 8-column piece q (of C's half and of dy)
    const int tp = tid & 31, q = tid >> 5;
    u32x4_t rc0, rc1, rd0, rd1;
    auto load = [&](int64_t k) {
        const int64_t t = k * kH0Q + 2 * tp;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        rc0 = rc1 = rd0 = rd1 = z;
        if (t < L) {
            rc0 = *reinterpret_cast<const u32x4_t*>(Cm + ((b * L + t) * G + g) * kH0N + kNh * nh + 8 * q);
            rd0 = *reinterpret_cast<const u32x4_t*>(dy + ((b * L + t) * H + h) * kH0P + 8 * q);
        }
        if (t + 1 < L) {
            rc1 = *reinterpret_cast<const u32x4_t*>(Cm + ((b * L + t + 1) * G + g) * kH0N + kNh * nh + 8 * q);
            rd1 = *reinterpret_cast<const u32x4_t*>(dy + ((b * L + t + 1) * H + h) * kH0P + 8 * q);
        }
    };
    // column 8 q + e of the pair: (token 2 tp, token 2 tp + 1) as one 4-byte word
    auto store = [&](int64_t k) {
        uint8_t* ct = sCt[k & 1];
        uint8_t* dv = sDy[k & 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = 16 * (e & 1);
            const uint32_t c2 = ((rc0[e >> 1] >> sh) & 0xFFFFu) | (((rc1[e >> 1] >> sh) & 0xFFFFu) << 16);
            const uint32_t d2 = ((rd0[e >> 1] >> sh) & 0xFFFFu) | (((rd1[e >> 1] >> sh) & 0xFFFFu) << 16);
            *reinterpret_cast<uint32_t*>(ct + (8 * q + e) * kH0Row + 4 * tp) = c2;
            *reinterpret_cast<uint32_t*>(dv + (8 * q + e) * kH0Row + 4 * tp) = d2;
        }
    };
    float offset = 0.0f;  // log2 of E at the end of the previous chunk (wave 0)
    bool alive = true;    // no sequence change so far (wave 0, uniform)
    // E_t of chunk k into sE[k & 1]; sStop[k & 1] = nothing after chunk k contributes
    auto scan_e = [&](int64_t k) {
        const int64_t t = k * kH0Q + lane;
        const bool in = t < L;
        const float v = in ? dt[(b * L + t) * H + h] * a2 : 0.0f;
        const float cum = h0_incl_sum(v);
        bool cut = false;  // a sequence change at or before this token (within the chunk)
        if (sq) {
            const bool chg = in && t > 0 && sq[t] != sq[t - 1];
            const uint64_t m = __ballot(chg);
            const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);  // lanes 0 .. lane
            cut = (m & upto) != 0;
        }
        const bool ok = alive && !cut && in;
        sE[k & 1][lane] = ok ? __builtin_amdgcn_exp2f(offset + cum) : 0.0f;
        offset += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), kH0Q - 1));
        const bool any_cut = __ballot(cut) != 0;
        alive = alive && !any_cut;
        const float e_end = __builtin_amdgcn_exp2f(offset);
        if (lane == 0) sStop[k & 1] = (!alive || e_end == 0.0f || k + 1 >= nchunks) ? 1 : 0;
    };
    f32x4_t acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (nchunks > 0) {
        load(0);
        store(0);
        if (wave == 0) scan_e(0);
    }
    __syncthreads();
    for (int64_t k = 0; k < nchunks; ++k) {
        const bool stop = sStop[k & 1] != 0;
        if (!stop) load(k + 1);
        const uint8_t* ct = sCt[k & 1];
        const uint8_t* dv = sDy[k & 1];
        // dh[p][n] += sum_t (E_t dy[t][p]) C[t][n]; lane: row p = 16 wave + li of the A
        // operand, tokens 32 ks + 8 g4 .. +7
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int tb = 32 * ks + 8 * g4;
            const f32x4_t e0 = *reinterpret_cast<const f32x4_t*>(&sE[k & 1][tb]);
            const f32x4_t e1 = *reinterpret_cast<const f32x4_t*>(&sE[k & 1][tb + 4]);
            const u32x4_t dw = *reinterpret_cast<const u32x4_t*>(dv + (16 * wave + li) * kH0Row + 2 * tb);
            float av[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ee = e < 4 ? e0[e] : e1[e - 4];
                const uint32_t bits = (dw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                av[e] = ee * __uint_as_float(bits << 16);
            }
            u32x4_t hv, lv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t hp = pack_bf16x2(av[2 * e], av[2 * e + 1]);
                hv[e] = hp;
                const float h0f = __uint_as_float(hp << 16), h1f = __uint_as_float(hp & 0xFFFF0000u);
                lv[e] = pack_bf16x2(av[2 * e] - h0f, av[2 * e + 1] - h1f);
            }
            const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, hv), alo = __builtin_bit_cast(bf16x8_t, lv);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(ct + (16 * n + li) * kH0Row + 2 * tb);
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, acc[n], 0, 0, 0);
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, acc[n], 0, 0, 0);
            }
        }
        if (stop) break;  // uniform: every thread read the same flag
        store(k + 1);     // the other buffer, last read before the previous barrier
        if (wave == 0) scan_e(k + 1);
        __syncthreads();
    }
    // the final state's term, E_{L-1} dF (zero after a sequence change or an underflow);
    // lane holds dh[p][n] for p = 16 wave + 4 g4 + r, n = 64 nh + 16 nt + li
    __shared__ float sEnd;
    __syncthreads();
    if (wave == 0 && lane == 0) sEnd = alive ? __builtin_amdgcn_exp2f(offset) : 0.0f;
    __syncthreads();
    const float eend = sEnd;
    float* out = dh0 + (b * H + h) * kH0P * kH0N;
    const float* fin = dfin ? dfin + (b * H + h) * kH0P * kH0N : nullptr;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int p = 16 * wave + 4 * g4 + rr, n = kNh * nh + 16 * nt + li;
            float v = acc[nt][rr];
            if (fin) v = __builtin_fmaf(eend, fin[p * kH0N + n], v);
            out[p * kH0N + n] = v;
        }
    }
}

// dh_{-1}, general shapes: one thread per (b, h, p, n), the token loop of the definition
// (stops at the first sequence change or once E underflows to 0)
template <class D>
__global__ void scan_bwd_h0_generic_kernel(const float* dt, const float* A,
                                           const typename D::T* Cm, const int32_t* seq,
                                           const typename D::T* dy, const float* dfin,
                                           float* dh0, int64_t B, int64_t L, int64_t H,
                                           int64_t P, int64_t G, int64_t N) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= B * H * P * N) return;
    const int64_t n = i % N, p = (i / N) % P, h = (i / (N * P)) % H, b = i / (N * P * H);
    const int64_t g = h / (H / G);
    const int32_t* sq = seq ? seq + b * L : nullptr;
    float e = 1.0f, acc = 0.0f;
    bool alive = true;
    for (int64_t t = 0; t < L; ++t) {
        if (sq && t > 0 && sq[t] != sq[t - 1]) {
            alive = false;
            break;
        }
        e *= __expf(dt[(b * L + t) * H + h] * A[h]);
        if (e == 0.0f) break;
        acc = __builtin_fmaf(D::load(dy, ((b * L + t) * H + h) * P + p) * e,
                             D::load(Cm, ((b * L + t) * G + g) * N + n), acc);
    }
    if (dfin && alive) acc = __builtin_fmaf(e, dfin[i], acc);
    dh0[i] = acc;
}

}  // namespace

int64_t conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t channels, int64_t width) {
    if (batch <= 0 || seqlen <= 0) return 0;
    const int64_t nruns = (seqlen + kConvBwdRun - 1) / kConvBwdRun;
    return batch * nruns * channels * (width + 1) * static_cast<int64_t>(sizeof(float));
}

hipError_t launch_conv1d_bwd(const void* x, const float* w, const float* bias, const void* init,
                             const int32_t* seq, const void* dy, const void* dfin, void* dx,
                             void* dinit, float* dw, float* dbias, void* workspace,
                             int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                             ssm_dtype_t dtype, ssm_act_t act, hipStream_t stream) {
    const int64_t C = channels, K = width;
    if (seqlen == 0) {
        const int64_t nst = batch * C * (K - 1);
        if (dinit && nst > 0) {
            const unsigned grid = static_cast<unsigned>((nst + 255) / 256);
            if (dtype == SSM_BF16)
                conv1d_bwd_empty_kernel<BF16><<<grid, 256, 0, stream>>>(
                    static_cast<const uint16_t*>(dfin), static_cast<uint16_t*>(dinit), nst);
            else
                conv1d_bwd_empty_kernel<F32><<<grid, 256, 0, stream>>>(
                    static_cast<const float*>(dfin), static_cast<float*>(dinit), nst);
        }
        fill_zero_f32_kernel<<<static_cast<unsigned>((C * K + 255) / 256), 256, 0, stream>>>(dw, C * K);
        if (dbias) fill_zero_f32_kernel<<<static_cast<unsigned>((C + 255) / 256), 256, 0, stream>>>(dbias, C);
        return hipGetLastError();
    }
    const int nruns = static_cast<int>((seqlen + kConvBwdRun - 1) / kConvBwdRun);
    dim3 grid(static_cast<unsigned>((C + kConvBwdThreads - 1) / kConvBwdThreads),
              static_cast<unsigned>(nruns), static_cast<unsigned>(batch));
    float* part = static_cast<float*>(workspace);
    const int silu = act == SSM_ACT_SILU ? 1 : 0;
#define SSM_CBWD(KK)                                                                           \
    case KK:                                                                                   \
        if (dtype == SSM_BF16)                                                                 \
            conv1d_bwd_kernel<BF16, KK><<<grid, kConvBwdThreads, 0, stream>>>(                 \
                static_cast<const uint16_t*>(x), w, bias, static_cast<const uint16_t*>(init),   \
                seq, static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(dfin),      \
                static_cast<uint16_t*>(dx), static_cast<uint16_t*>(dinit), part, seqlen, C,     \
                nruns, silu);                                                                  \
        else                                                                                   \
            conv1d_bwd_kernel<F32, KK><<<grid, kConvBwdThreads, 0, stream>>>(                  \
                static_cast<const float*>(x), w, bias, static_cast<const float*>(init), seq,    \
                static_cast<const float*>(dy), static_cast<const float*>(dfin),                \
                static_cast<float*>(dx), static_cast<float*>(dinit), part, seqlen, C, nruns,    \
                silu);                                                                         \
        break;
    constexpr int kVec = 2;  // channels per thread of the bf16 vector kernel
    const bool vec = dtype == SSM_BF16 && C % kVec == 0 &&
                     ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(dy) |
                       reinterpret_cast<uintptr_t>(dx)) & (2 * kVec - 1)) == 0;
    if (vec) {
        const dim3 grid4(static_cast<unsigned>((C / kVec + 63) / 64),
                         static_cast<unsigned>((nruns + 3) / 4), static_cast<unsigned>(batch));
#define SSM_CBWD4(KK)                                                                          \
    case KK:                                                                                   \
        conv1d_bwd_bf16vec_kernel<KK, kVec><<<grid4, kConvBwdThreads, 0, stream>>>(            \
            static_cast<const uint16_t*>(x), w, bias, static_cast<const uint16_t*>(init), seq,  \
            static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(dfin),              \
            static_cast<uint16_t*>(dx), static_cast<uint16_t*>(dinit), part, seqlen, C, nruns, \
            silu);                                                                             \
        break;
        switch (K) {
            SSM_CBWD4(2) SSM_CBWD4(3) SSM_CBWD4(4) SSM_CBWD4(5) SSM_CBWD4(6) SSM_CBWD4(7) SSM_CBWD4(8)
            default: return hipErrorInvalidValue;
        }
#undef SSM_CBWD4
    } else {
        switch (K) {
            SSM_CBWD(2) SSM_CBWD(3) SSM_CBWD(4) SSM_CBWD(5) SSM_CBWD(6) SSM_CBWD(7) SSM_CBWD(8)
            default: return hipErrorInvalidValue;
        }
    }
#undef SSM_CBWD
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nred = C * (K + 1);
    // the vector kernel leaves one partial per group of four runs
    const int64_t nparts = vec ? batch * ((nruns + 3) / 4) : batch * nruns;
    conv1d_bwd_reduce_kernel<<<static_cast<unsigned>((nred + 63) / 64), 256, 0, stream>>>(
        part, dw, dbias, C, static_cast<int>(K), nparts);
    return hipGetLastError();
}

hipError_t launch_scan_bwd_h0(const float* dt, const float* A, const void* Cm,
                              const int32_t* seq, const void* dy, const float* dfin, float* dh0,
                              int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t ngroups, int64_t dstate, ssm_dtype_t dtype,
                              hipStream_t stream) {
    const bool a16 = (reinterpret_cast<uintptr_t>(Cm) % 16) == 0 && (reinterpret_cast<uintptr_t>(dy) % 16) == 0;
    if (dtype == SSM_BF16 && headdim == kH0P && dstate == kH0N && a16 && seqlen > 0) {
        dim3 grid(static_cast<unsigned>(nheads), static_cast<unsigned>(batch), 2);  // z: column half
        scan_bwd_h0_mfma_kernel<<<grid, 256, 0, stream>>>(
            dt, A, static_cast<const uint16_t*>(Cm), seq, static_cast<const uint16_t*>(dy), dfin,
            dh0, seqlen, nheads, ngroups);
        return hipGetLastError();
    }
    const int64_t n = batch * nheads * headdim * dstate;
    const unsigned grid = static_cast<unsigned>((n + 255) / 256);
    if (dtype == SSM_BF16)
        scan_bwd_h0_generic_kernel<BF16><<<grid, 256, 0, stream>>>(
            dt, A, static_cast<const uint16_t*>(Cm), seq, static_cast<const uint16_t*>(dy), dfin,
            dh0, batch, seqlen, nheads, headdim, ngroups, dstate);
    else
        scan_bwd_h0_generic_kernel<F32><<<grid, 256, 0, stream>>>(
            dt, A, static_cast<const float*>(Cm), seq, static_cast<const float*>(dy), dfin, dh0,
            batch, seqlen, nheads, headdim, ngroups, dstate);
    return hipGetLastError();
}

}  // namespace ssm
