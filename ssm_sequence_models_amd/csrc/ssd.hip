// ssd.hip -- chunked ("state-space dual") form of the selective scan on gfx950 MFMA, with the
// causal conv1d front end fused in.  bf16 activations, headdim 64, dstate 128, chunk 64.
//
// What is computed is the recurrence of the length-generalization reading notes, Sec. 2.1
// Eq. (1), started from the initial state h_{-1} (Sec. 2.5 Eq. (4)) and returning the final
// state (Sec. 2.6 State Passing); the conv is the extended-sequence definition of the
// causal-conv1d tutorial ch. 7.  Eq. (4) restricted to one chunk of Q tokens gives, with
// cum_i = sum_{tau<=i} dt_tau A_h inside the chunk (the transition taken in log space, as
// Sec. 2.5 notes for the diagonal case):
//     y_i     = sum_{j<=i} (C_i . B_j) exp(cum_i - cum_j) dt_j x_j      (intra-chunk part)
//             + exp(cum_i) C_i . h_prev                                  (initial-state part)
//     h_next  = exp(cum_{Q-1}) h_prev + sum_j exp(cum_{Q-1} - cum_j) dt_j x_j B_j^T
// Every exp argument is a difference cum_i - cum_j <= 0, so nothing overflows; underflow to
// 0 is the exact limit.  A packed-sequence boundary inside the chunk cuts the sums at the
// last reset (the state restarts from zero there).
//
// Work split:
//  * ssd_prep_kernel, one block per (batch row, chunk, group): runs the conv (+phi, bf16
//    rounding) over the chunk's B and C channels once for all heads of the group and writes
//    C (token-major), B (channel-major) and G = C B^T (fp32, MFMA) to the workspace.  Doing
//    this per head would repeat the B/C conv nheads times.
//  * ssd_main_kernel, one block per (batch row, head), 4 wavefronts, each owning 16 of the
//    64 head channels: it streams the head's x channels through the register-window conv,
//    keeps its [16 x 128] slice of the fp32 state in MFMA accumulators for the whole
//    sequence, and per chunk issues the three contractions on v_mfma_f32_16x16x32_bf16:
//        Y^T   += h^T-slice x C^T           (initial-state part)
//        Y^T   += X^T x M^T                 (intra-chunk part, M = G o decay mask)
//        h^T   += B^T x (W o X)             (state update)
//    The fp32 operands (h, M, W o X) enter as a hi + lo pair of bf16 (v = hi + lo with
//    |v - hi - lo| <= 2^-17 |v|); the other operand (x, B, C) is exact in bf16, so each
//    contraction is accurate to about fp32 while running at the bf16 MFMA rate.
//  * the next chunk's x / B / C / G tiles are fetched into registers while the current
//    chunk computes and dropped into the other half of a double-buffered LDS stage.
#include "internal.h"

namespace ssm {
namespace {

constexpr int kQ = 64;       // tokens per chunk
constexpr int kP = 64;       // head channels (4 waves x 16)
constexpr int kN = 128;      // state size
constexpr int kKmax = 8;     // widest conv handled
constexpr int kThreads = 256;
constexpr int kRowsMax = kQ + kKmax - 1;  // staged x rows incl. the conv halo

// LDS strides (bytes); +16 breaks power-of-two row strides
constexpr int kXStride = kP * 2 + 16;    // x rows [token][channel] bf16
constexpr int kCStride = kN * 2 + 16;    // C rows [token][n] bf16
constexpr int kBtStride = kQ * 2 + 16;   // B^T rows [n][token] bf16
constexpr int kMStride = kQ * 2 + 16;    // M rows [i][j] bf16

constexpr int kXBytes = ((kRowsMax * kXStride + 255) / 256) * 256;
constexpr int kCBytes = kQ * kCStride;
constexpr int kBtBytes = kN * kBtStride;
constexpr int kSeqBytes = ((kRowsMax * 4 + 15) / 16) * 16;
constexpr int kStageBytes = kXBytes + kCBytes + kBtBytes + kSeqBytes;
constexpr int kMBytes = kQ * kMStride;
constexpr int kScalarBytes = 5 * kQ * 4 + 16;
constexpr int kMainLds = 2 * kStageBytes + 2 * kMBytes + kScalarBytes;
static_assert(kMainLds <= 160 * 1024, "LDS budget");

// workspace per (row, chunk, group)
constexpr int64_t kWsC = static_cast<int64_t>(kQ) * kN;    // bf16 elements
constexpr int64_t kWsBt = static_cast<int64_t>(kN) * kQ;   // bf16 elements
constexpr int64_t kWsG = static_cast<int64_t>(kQ) * kQ;    // fp32 elements

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint8_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// v = hi + lo, hi = rne(v), lo = rne(v - hi)
__device__ __forceinline__ void split_hilo(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(v[e]);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
    }
}

__device__ __forceinline__ float warp_incl_sum(float v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}
__device__ __forceinline__ int warp_incl_max(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off);
        if (lane >= off) v = max(v, o);
    }
    return v;
}

__device__ __forceinline__ int64_t ws_base(const ChunkedArgs& a, int64_t b, int64_t c,
                                           int64_t g, int64_t nC) {
    return (b * nC + c) * a.G + g;
}

// conv of one channel over 8 consecutive outputs, rounded to bf16 as the exact value rounds
// (double sums: the products of fp32 weights and bf16 inputs are exact); u[0 .. 8+K-2] are
// the inputs of the window starting K-1 before the first output, ids likewise (a tap counts
// only if its id equals the output token's)
template <bool HAS_SEQ>
__device__ __forceinline__ void conv8(const double (&u)[kKmax + 7], const int32_t (&id)[kKmax + 7],
                                      const double (&w)[kKmax], double bias, int K, int act,
                                      uint16_t (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        double z = bias;
        int32_t idc = 0;
        if (HAS_SEQ) {
#pragma unroll
            for (int k = 0; k < kKmax; ++k)
                if (k == K - 1) idc = id[e + k];
        }
#pragma unroll
        for (int k = 0; k < kKmax; ++k) {
            if (k < K) {
                const double tap = (!HAS_SEQ || id[e + k] == idc) ? u[e + k] : 0.0;
                z = fma(w[k], tap, z);
            }
        }
        out[e] = act_to_bf16(z, act);
    }
}

// =======================================================================================
// prep: conv + bf16 rounding of the B / C channels of one (row, chunk, group), then
// C token-major, B channel-major and G = C B^T into the workspace
// =======================================================================================
__global__ void __launch_bounds__(kThreads)
ssd_prep_kernel(ChunkedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[2 * kQ * kCStride + kSeqBytes];
    uint8_t* sB = sm;                 // [token][n] bf16
    uint8_t* sC = sm + kQ * kCStride; // [token][n] bf16
    int32_t* sSeq = reinterpret_cast<int32_t*>(sm + 2 * kQ * kCStride);

    const int tid = threadIdx.x;
    const int64_t cn = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int64_t L = a.L, K = a.K;
    const int64_t nC = (L + kQ - 1) / kQ;
    const int64_t t0 = cn * kQ;
    const bool has_seq = a.seq_idx != nullptr;

    if (has_seq && tid < kQ + K - 1) {
        int64_t t = t0 - (K - 1) + tid;
        t = t < 0 ? 0 : (t >= L ? L - 1 : t);
        sSeq[tid] = a.seq_idx[b * L + t];
    }
    __syncthreads();

    for (int ch = tid; ch < 2 * kN; ch += kThreads) {
        const bool isC = ch >= kN;
        const int n = isC ? ch - kN : ch;
        const uint16_t* src = isC ? a.csrc : a.bsrc;
        const int64_t row = isC ? a.c_row : a.b_row;
        const int64_t col = (isC ? a.c_col0 : a.b_col0) + g * kN + n;
        uint8_t* dst = isC ? sC : sB;
        if (a.fused_conv) {
            double w[kKmax];
#pragma unroll
            for (int k = 0; k < kKmax; ++k) w[k] = k < K ? a.conv_w[col * K + k] : 0.0f;
            const double bias = a.conv_b ? a.conv_b[col] : 0.0f;
            // sliding window: win[kKmax-1-(K-1) ..] oldest -> newest; idw likewise
            double win[kKmax];
            int32_t idw[kKmax];
#pragma unroll
            for (int k = 0; k < kKmax; ++k) { win[k] = 0.0; idw[k] = 0; }
#pragma unroll
            for (int k = 0; k < kKmax - 1; ++k) {
                const int64_t tau = k - (kKmax - 1 - (K - 1));  // 0 .. K-2 for live slots
                if (tau >= 0) {
                    const int64_t t = t0 - (K - 1) + tau;
                    float v = 0.0f;
                    if (t >= 0)
                        v = bf16_to_f32(src[(b * L + t) * row + col]);
                    else if (a.conv_init)
                        v = bf16_to_f32(a.conv_init[(b * a.C_conv + col) * (K - 1) + (K - 1) + t]);
                    win[k] = v;
                    idw[k] = has_seq ? sSeq[tau] : 0;
                }
            }
            for (int j = 0; j < kQ; ++j) {
                const int64_t t = t0 + j;
                const double xv = t < L ? bf16_to_f32(src[(b * L + t) * row + col]) : 0.0f;
                const int32_t idt = has_seq ? sSeq[j + K - 1] : 0;
                win[kKmax - 1] = xv;
                idw[kKmax - 1] = idt;
                double z = bias;
#pragma unroll
                for (int k = 0; k < kKmax; ++k) {
                    const int kk = k - (kKmax - K);  // tap index 0 .. K-1 for live slots
                    if (kk >= 0) {
                        const double tap = (!has_seq || idw[k] == idt) ? win[k] : 0.0;
                        z = fma(w[kk], tap, z);
                    }
                }
                const uint16_t v = t < L ? act_to_bf16(z, a.act) : uint16_t(0);
                *reinterpret_cast<uint16_t*>(dst + j * kCStride + n * 2) = v;
#pragma unroll
                for (int k = 0; k < kKmax - 1; ++k) { win[k] = win[k + 1]; idw[k] = idw[k + 1]; }
            }
        } else {
            for (int j = 0; j < kQ; ++j) {
                const int64_t t = t0 + j;
                const uint16_t v = t < L ? src[(b * L + t) * row + col] : uint16_t(0);
                *reinterpret_cast<uint16_t*>(dst + j * kCStride + n * 2) = v;
            }
        }
    }
    __syncthreads();

    const int64_t base = ws_base(a, b, cn, g, nC);
    uint16_t* wsC = static_cast<uint16_t*>(a.workspace);
    uint16_t* wsBt = wsC + a.B * nC * a.G * kWsC;
    float* wsG = reinterpret_cast<float*>(wsBt + a.B * nC * a.G * kWsBt);
    // C token-major: 16-byte pieces
    for (int idx = tid; idx < kQ * kN / 8; idx += kThreads) {
        const int i = idx >> 4, q = idx & 15;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sC + i * kCStride + q * 16);
        *reinterpret_cast<u32x4*>(wsC + base * kWsC + i * kN + q * 8) = v;
    }
    // B channel-major: gather 8 tokens of one channel
    for (int idx = tid; idx < kN * kQ / 8; idx += kThreads) {
        const int n = idx >> 3, jq = idx & 7;
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = *reinterpret_cast<const uint16_t*>(sB + (8 * jq + 2 * e) * kCStride + n * 2);
            const uint32_t hi = *reinterpret_cast<const uint16_t*>(sB + (8 * jq + 2 * e + 1) * kCStride + n * 2);
            w4[e] = lo | (hi << 16);
        }
        u32x4 v = {w4[0], w4[1], w4[2], w4[3]};
        *reinterpret_cast<u32x4*>(wsBt + base * kWsBt + n * kQ + jq * 8) = v;
    }
    // G = C B^T for the tiles on or below the diagonal; wave w owns rows 16w .. 16w+15
    const int wave = tid >> 6, lane = tid & 63, li = lane & 15, g4 = lane >> 4;
    for (int jt = 0; jt <= wave; ++jt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < kN / 32; ++m) {
            const bf16x8 av = lds_bf16x8(sC + (16 * wave + li) * kCStride + (32 * m + 8 * g4) * 2);
            const bf16x8 bv = lds_bf16x8(sB + (16 * jt + li) * kCStride + (32 * m + 8 * g4) * 2);
            acc = mfma(av, bv, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wsG[base * kWsG + (16 * wave + 4 * g4 + r) * kQ + 16 * jt + li] = acc[r];
    }
}

// =======================================================================================
// main kernel
// =======================================================================================
struct Stage {
    u32x4 x[3];
    u32x4 c[4];
    u32x4 bt[4];
    f32x4 gm[4];
    int32_t seq;
    float dt;
};

__device__ __forceinline__ void stage_load(const ChunkedArgs& a, int64_t b, int64_t h,
                                           int64_t g, int64_t cn, int64_t nC, int tid,
                                           Stage& s) {
    const int64_t L = a.L, K = a.K;
    const int rows = static_cast<int>(kQ + K - 1);
    const int64_t t0 = cn * kQ;
    // x rows (raw, pre-conv), 8 channels per piece
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int idx = tid + k * kThreads;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (idx < rows * 8) {
            const int rho = idx >> 3, q = idx & 7;
            const int64_t t = t0 - (K - 1) + rho;
            const int64_t col = a.x_col0 + h * kP + q * 8;
            if (t >= 0 && t < L) {
                v = *reinterpret_cast<const u32x4*>(a.x + (b * L + t) * a.x_row + col);
            } else if (t < 0 && a.fused_conv && a.conv_init) {
                uint32_t w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = a.conv_init[(b * a.C_conv + col + 2 * e) * (K - 1) + (K - 1) + t];
                    const uint32_t hi = a.conv_init[(b * a.C_conv + col + 2 * e + 1) * (K - 1) + (K - 1) + t];
                    w4[e] = lo | (hi << 16);
                }
                v = u32x4{w4[0], w4[1], w4[2], w4[3]};
            }
        }
        s.x[k] = v;
    }
    const int64_t base = ws_base(a, b, cn, g, nC);
    const uint16_t* wsC = static_cast<const uint16_t*>(a.workspace);
    const uint16_t* wsBt = wsC + a.B * nC * a.G * kWsC;
    const float* wsG = reinterpret_cast<const float*>(wsBt + a.B * nC * a.G * kWsBt);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + k * kThreads;
        s.c[k] = *reinterpret_cast<const u32x4*>(wsC + base * kWsC + idx * 8);
        s.bt[k] = *reinterpret_cast<const u32x4*>(wsBt + base * kWsBt + idx * 8);
    }
    {
        const int i = tid >> 2, jb = (tid & 3) * 16;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (jb <= i) v = *reinterpret_cast<const f32x4*>(wsG + base * kWsG + i * kQ + jb + 4 * k);
            s.gm[k] = v;
        }
    }
    s.seq = 0;
    if (a.seq_idx && tid < rows) {
        int64_t t = t0 - (K - 1) + tid;
        t = t < 0 ? 0 : (t >= L ? L - 1 : t);
        s.seq = a.seq_idx[b * L + t];
    }
    s.dt = 0.0f;
    if (tid < kQ && t0 + tid < L) s.dt = a.dt[(b * L + t0 + tid) * a.H + h];
}

__device__ __forceinline__ void stage_store(uint8_t* stage, const Stage& s, int tid, int rows) {
    uint8_t* sX = stage;
    uint8_t* sC = stage + kXBytes;
    uint8_t* sBt = sC + kCBytes;
    int32_t* sSeq = reinterpret_cast<int32_t*>(sBt + kBtBytes);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int idx = tid + k * kThreads;
        if (idx < rows * 8) {
            const int rho = idx >> 3, q = idx & 7;
            *reinterpret_cast<u32x4*>(sX + rho * kXStride + q * 16) = s.x[k];
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + k * kThreads;
        const int i = idx >> 4, q = idx & 15;
        *reinterpret_cast<u32x4*>(sC + i * kCStride + q * 16) = s.c[k];
        const int n = idx >> 3, jq = idx & 7;
        *reinterpret_cast<u32x4*>(sBt + n * kBtStride + jq * 16) = s.bt[k];
    }
    if (tid < rows) sSeq[tid] = s.seq;
}

template <bool FUSED, bool HAS_SEQ>
__global__ void __launch_bounds__(kThreads, 1)
ssd_main_kernel(ChunkedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[kMainLds];
    uint8_t* stages = sm;
    uint8_t* sMhi = sm + 2 * kStageBytes;
    uint8_t* sMlo = sMhi + kMBytes;
    float* sCum = reinterpret_cast<float*>(sMlo + kMBytes);
    float* sDtv = sCum + kQ;
    int32_t* sR = reinterpret_cast<int32_t*>(sDtv + kQ);
    float* sW = reinterpret_cast<float*>(sR + kQ);
    float* sE = sW + kQ;
    float* sDecay = sE + kQ;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, li = lane & 15, g4 = lane >> 4;

    // block -> (row, head): consecutive units on one XCD (blocks are dealt round-robin over
    // the 8 XCDs), so the heads of one row share that XCD's L2 for the B/C/G tiles
    const int64_t nblk = gridDim.x;
    const int64_t k = blockIdx.x;
    const int64_t u = (nblk % 8 == 0) ? (k % 8) * (nblk / 8) + k / 8 : k;
    const int64_t b = u / a.H, h = u % a.H;
    const int64_t g = h / (a.H / a.G);
    const int64_t L = a.L, K = a.K;
    const int rows = static_cast<int>(kQ + K - 1);
    const int64_t nC = (L + kQ - 1) / kQ;
    const float Ah = a.A[h];
    const int p_own = 16 * wave + li;  // channel whose x this lane convolves / owns in h

    // conv weights of this lane's channel
    double cw[kKmax];
    double cbias = 0.0;
    if (FUSED) {
        const int64_t cc = a.x_col0 + h * kP + p_own;
#pragma unroll
        for (int kk = 0; kk < kKmax; ++kk) cw[kk] = kk < K ? a.conv_w[cc * K + kk] : 0.0f;
        cbias = a.conv_b ? a.conv_b[cc] : 0.0f;
    }

    // state slice: acc[t][r] = h[p_own][n(t, 4*g4 + r)], n(t, rho) = 32(t/2) + 8(rho/4) +
    // 4(t%2) + rho%4, i.e. for k-step m the lane holds n = 32m + 8*g4 + e, e = 0..7
    f32x4 acc[8];
    {
        const float* src = a.init_state ? a.init_state + ((b * a.H + h) * kP + p_own) * kN : nullptr;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 v0 = {0.0f, 0.0f, 0.0f, 0.0f}, v1 = v0;
            if (src) {
                v0 = *reinterpret_cast<const f32x4*>(src + 32 * m + 8 * g4);
                v1 = *reinterpret_cast<const f32x4*>(src + 32 * m + 8 * g4 + 4);
            }
            acc[2 * m] = v0;
            acc[2 * m + 1] = v1;
        }
    }

    Stage st;
    stage_load(a, b, h, g, 0, nC, tid, st);
    stage_store(stages, st, tid, rows);
    f32x4 gm[4] = {st.gm[0], st.gm[1], st.gm[2], st.gm[3]};
    float dt_cur = st.dt;
    __syncthreads();

    for (int64_t cn = 0; cn < nC; ++cn) {
        uint8_t* stage = stages + (cn & 1) * kStageBytes;
        const uint8_t* sX = stage;
        const uint8_t* sC = stage + kXBytes;
        const uint8_t* sBt = sC + kCBytes;
        const int32_t* sSeq = reinterpret_cast<const int32_t*>(sBt + kBtBytes);
        const int64_t t0 = cn * kQ;
        const bool more = cn + 1 < nC;
        if (more) stage_load(a, b, h, g, cn + 1, nC, tid, st);

        // ---- chunk scalars (wave 0, lane = token) ----
        if (wave == 0) {
            const int j = lane;
            const bool valid = t0 + j < L;
            const float dtv = valid ? dt_cur : 0.0f;
            const float cum = warp_incl_sum(dtv * Ah, lane);
            int rst = -1;
            if (HAS_SEQ && valid && t0 + j > 0 && sSeq[j + K - 1] != sSeq[j + K - 2]) rst = j;
            const int r = warp_incl_max(rst, lane);
            const float cum_last = __shfl(cum, kQ - 1);
            const int r_last = __shfl(r, kQ - 1);
            sCum[j] = cum;
            sDtv[j] = dtv;
            sR[j] = r;
            sE[j] = r < 0 ? __expf(cum) : 0.0f;
            sW[j] = j >= r_last ? __expf(cum_last - cum) * dtv : 0.0f;
            if (j == 0) *sDecay = r_last < 0 ? __expf(cum_last) : 0.0f;
        }

        // ---- conv of this lane's channel over its 16 tokens (j = 32s + 8*g4 + e) ----
        bf16x8 xv[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int j0 = 32 * s + 8 * g4;
            if (FUSED) {
                double u[kKmax + 7];
                int32_t id[kKmax + 7];
#pragma unroll
                for (int tau = 0; tau < kKmax + 7; ++tau) {
                    if (tau < 8 + K - 1) {
                        u[tau] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sX + (j0 + tau) * kXStride + p_own * 2));
                        id[tau] = HAS_SEQ ? sSeq[j0 + tau] : 0;
                    } else {
                        u[tau] = 0.0;
                        id[tau] = 0;
                    }
                }
                uint16_t o[8];
                conv8<HAS_SEQ>(u, id, cw, cbias, static_cast<int>(K), a.act, o);
#pragma unroll
                for (int e = 0; e < 8; ++e) xv[s][e] = __builtin_bit_cast(__bf16, o[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t raw = *reinterpret_cast<const uint16_t*>(sX + (j0 + e + K - 1) * kXStride + p_own * 2);
                    xv[s][e] = __builtin_bit_cast(__bf16, raw);
                }
            }
        }
        __syncthreads();  // scalars visible

        // ---- M = G o exp(cum_i - cum_j) dt_j on j <= i within the segment; hi/lo -> LDS ----
        {
            const int i = tid >> 2, jb = (tid & 3) * 16;
            float mv[16];
            if (jb <= i) {
                const float ci = sCum[i];
                const int ri = sR[i];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = jb + e;
                    const float gv = gm[e >> 2][e & 3];
                    const float m = gv * __expf(ci - sCum[j]) * sDtv[j];
                    mv[e] = (j <= i && j >= ri) ? m : 0.0f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) mv[e] = 0.0f;
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float v8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v8[e] = mv[8 * half + e];
                bf16x8 hi, lo;
                split_hilo(v8, hi, lo);
                *reinterpret_cast<bf16x8*>(sMhi + i * kMStride + (jb + 8 * half) * 2) = hi;
                *reinterpret_cast<bf16x8*>(sMlo + i * kMStride + (jb + 8 * half) * 2) = lo;
            }
        }
        // per-lane scalars for the contractions (read before the next barrier: wave 0
        // rewrites them for the next chunk right after it)
        float eI[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) eI[I] = sE[16 * I + li];
        float wj[2][8];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) wj[s][e] = sW[32 * s + 8 * g4 + e];
        const float decay = *sDecay;
        __syncthreads();  // M visible

        // ---- Y^T[p][i] (p = 16*wave + 4*g4 + r, i = 16I + li) ----
        f32x4 yo[4], yi[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            yo[I] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            yi[I] = yo[I];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float hv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hv[e] = acc[2 * m][e];
                hv[4 + e] = acc[2 * m + 1][e];
            }
            bf16x8 hhi, hlo;
            split_hilo(hv, hhi, hlo);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const bf16x8 cv = lds_bf16x8(sC + (16 * I + li) * kCStride + (32 * m + 8 * g4) * 2);
                yo[I] = mfma(hhi, cv, yo[I]);
                yo[I] = mfma(hlo, cv, yo[I]);
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (32 * s <= 16 * I + 15) {
                    const bf16x8 mh = lds_bf16x8(sMhi + (16 * I + li) * kMStride + (32 * s + 8 * g4) * 2);
                    const bf16x8 ml = lds_bf16x8(sMlo + (16 * I + li) * kMStride + (32 * s + 8 * g4) * 2);
                    yi[I] = mfma(xv[s], mh, yi[I]);
                    yi[I] = mfma(xv[s], ml, yi[I]);
                }
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const int64_t t = t0 + 16 * I + li;
            if (t < L) {
                uint2 pk;
                pk.x = pack_bf16x2(eI[I] * yo[I][0] + yi[I][0], eI[I] * yo[I][1] + yi[I][1]);
                pk.y = pack_bf16x2(eI[I] * yo[I][2] + yi[I][2], eI[I] * yo[I][3] + yi[I][3]);
                *reinterpret_cast<uint2*>(a.y + ((b * L + t) * a.H + h) * kP + 16 * wave + 4 * g4) = pk;
            }
        }

        // ---- state update: h^T[n][p] = decay h^T + B^T (W o X) ----
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] *= decay;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float wx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wx[e] = wj[s][e] * static_cast<float>(xv[s][e]);
            bf16x8 bh, bl;
            split_hilo(wx, bh, bl);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int n_row = 32 * (t >> 1) + 8 * (li >> 2) + 4 * (t & 1) + (li & 3);
                const bf16x8 bv = lds_bf16x8(sBt + n_row * kBtStride + (32 * s + 8 * g4) * 2);
                acc[t] = mfma(bv, bh, acc[t]);
                acc[t] = mfma(bv, bl, acc[t]);
            }
        }

        // ---- next chunk's tiles into the other stage ----
        if (more) {
            stage_store(stages + ((cn + 1) & 1) * kStageBytes, st, tid, rows);
#pragma unroll
            for (int q = 0; q < 4; ++q) gm[q] = st.gm[q];
            dt_cur = st.dt;
        }
        __syncthreads();
    }

    // ---- final SSM state ----
    if (a.final_state) {
        float* dst = a.final_state + ((b * a.H + h) * kP + p_own) * kN;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            *reinterpret_cast<f32x4*>(dst + 32 * m + 8 * g4) = acc[2 * m];
            *reinterpret_cast<f32x4*>(dst + 32 * m + 8 * g4 + 4) = acc[2 * m + 1];
        }
    }
    // ---- final conv state F = u[L .. L+K-2] for this head's x channels and for slice h of
    // the B / C channels: all reads first, then a barrier, then the writes, so an in-place
    // state pair is never read after being overwritten ----
    if (FUSED && a.conv_final) {
        const int64_t km1 = K - 1;
        const int64_t nx = kP * km1;
        const int64_t nbc_all = 2 * a.G * kN * km1;
        const int64_t per = (nbc_all + a.H - 1) / a.H;
        const int64_t bc_lo = min(h * per, nbc_all), bc_hi = min((h + 1) * per, nbc_all);
        const int64_t total = nx + (bc_hi - bc_lo);
        constexpr int kMaxItems = 12;  // >= ceil((64*7 + 2*128*7) / 256) for every G <= H
        uint16_t fv[kMaxItems];
        int64_t fidx[kMaxItems];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < kMaxItems; ++q) {
            const int64_t idx = tid + static_cast<int64_t>(q) * kThreads;
            if (idx < total) {
                int64_t cc, r;
                if (idx < nx) {
                    cc = a.x_col0 + h * kP + idx / km1;
                    r = idx % km1;
                } else {
                    const int64_t e = bc_lo + (idx - nx);
                    cc = a.b_col0 + e / km1;  // B then C channels, contiguous in xBC
                    r = e % km1;
                }
                const int64_t mpos = L + r;
                uint16_t v;
                if (mpos < km1)
                    v = a.conv_init ? a.conv_init[(b * a.C_conv + cc) * km1 + mpos] : uint16_t(0);
                else
                    v = a.x[(b * L + (mpos - km1)) * a.x_row + cc];
                fv[q] = v;
                fidx[q] = (b * a.C_conv + cc) * km1 + r;
                cnt = q + 1;
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kMaxItems; ++q)
            if (q < cnt) a.conv_final[fidx[q]] = fv[q];
    }
}

}  // namespace

bool chunked_supported(int64_t P, int64_t N, ssm_dtype_t dtype) {
    return dtype == SSM_BF16 && P == kP && N == kN;
}

size_t chunked_workspace_bytes(int64_t B, int64_t L, int64_t G, int64_t N) {
    if (N != kN) return 0;
    const int64_t nC = (L + kQ - 1) / kQ;
    const int64_t units = B * nC * G;
    return static_cast<size_t>(units * (kWsC * 2 + kWsBt * 2 + kWsG * 4));
}

hipError_t launch_chunked(const ChunkedArgs& a, hipStream_t stream, hipEvent_t ev_before_main,
                          hipEvent_t ev_after_main) {
    if (a.B == 0 || a.L == 0) return hipSuccess;
    const int64_t nC = (a.L + kQ - 1) / kQ;
    ssd_prep_kernel<<<dim3(static_cast<unsigned>(nC), static_cast<unsigned>(a.G),
                           static_cast<unsigned>(a.B)),
                      kThreads, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_before_main) hipEventRecord(ev_before_main, stream);
    const dim3 grid(static_cast<unsigned>(a.B * a.H));
    const bool seq = a.seq_idx != nullptr;
    if (a.fused_conv) {
        if (seq) ssd_main_kernel<true, true><<<grid, kThreads, 0, stream>>>(a);
        else ssd_main_kernel<true, false><<<grid, kThreads, 0, stream>>>(a);
    } else {
        if (seq) ssd_main_kernel<false, true><<<grid, kThreads, 0, stream>>>(a);
        else ssd_main_kernel<false, false><<<grid, kThreads, 0, stream>>>(a);
    }
    e = hipGetLastError();
    if (ev_after_main) hipEventRecord(ev_after_main, stream);
    return e;
}

}  // namespace ssm
