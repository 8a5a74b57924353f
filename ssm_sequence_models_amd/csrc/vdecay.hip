// vdecay.hip -- the scan with a diagonal transition (one decay per state dimension) for long
// rows: length-generalization reading notes, Sec. 2.1 Eq. (1) with A_t = diag(a_t) and
// Sec. 2.5's diagonal case (the transition taken from log coefficients), per head h, channel
// p and state dimension n:
//     state[p][n] <- a_t[n] state[p][n] + u_t x_t[p] B_t[n],    y_t[p] = C_t . state[p][:]
// with log a_t[n] = log_decay[b][t][h][n] or dt_t A_vec[h][n], u_t = dt_t (or 1).
//
// Token-sequential, laid out for issue rate rather than for the decode step's one token:
//   - one block per (row, head, half of the head's 64 channels), 512 threads: waves 0-3
//     compute, waves 4-7 stage.  Two blocks share a CU, so each SIMD runs two compute waves
//     and one hides the other's LDS and DPP latency;
//   - a compute lane owns a 2 x NL block of the state (channels p0, p0 + 1 with
//     p0 = 32 half + 2 (tid / 16), dimensions n = NL (tid % 16) .. +NL-1, NL = N / 16) in
//     registers for the whole row.  Per token it reads its NL values of B, C and a_t and 2 of
//     x from LDS (lanes sharing them read the same addresses), issues 2 NL decay multiplies,
//     2 NL input accumulates and 2 NL read-out accumulates, and a reduce-scatter over the 16
//     lanes of its channel block leaves y_t[p] of one channel in every eighth lane.  The
//     reduce-scatter of a token runs in the next token's iteration, where nothing depends on
//     it, so its exchange latency overlaps that token's updates;
//   - the staging waves copy a tile of 16 tokens (B, C, the block's x, dt, and
//     a_t[n] = exp(log a_t[n]), formed once per token and dimension; a_t = 0 where seq_idx
//     starts a new sequence, which is the reset) into one of two LDS buffers while the
//     compute waves consume the other.  A staging thread moves one (token, 8 dimensions)
//     piece with 16-byte loads, and issues tile k+2's loads as soon as it has stored tile
//     k+1, so they have a whole tile of compute to arrive; one barrier per tile.
// Measured at the 1.3B-like shape (B 4, L 8192, 64 heads, gates [B, L, H, N]): one block per
// (row, head) with a quarter row per lane 4.6 ms (LDS-return bound at 24 reads per token);
// 4 x 8 blocks per lane 4.1 ms, 3.37 ms with batched staging loads, 3.31 ms with the
// pipelined reduce-scatter (compute alone 2.54 ms: one compute wave per SIMD leaves every
// latency exposed); pairing tokens under one reduce-scatter 5.5 ms (139 VGPRs); all eight
// waves computing 4 x 4 blocks with a 32-lane ds_swizzle reduction 3.65-3.80 ms; this
// layout, halves of the channels in two blocks per CU, 2.75 ms; quarters (one channel per
// lane, four blocks per (row, head) re-staging the same gates) 4.9 ms; one block per (row,
// head) with eight compute and four staging waves (no gate re-staging) 3.2 ms.  With staging
// switched off (work copy) the halves took 1.97 ms against 2.65: staging was not hidden;
// 16-byte staging loads issued a tile ahead took the call to 2.37 ms.  In this layout, 4 x 4
// blocks per lane (four LDS reads per token instead of seven, a 32-lane reduce-scatter with
// one ds_swizzle level) ran 2.25 ms against 2.13 for 2 x 8 blocks, timed side by side.
// Raising the compute or the staging waves' issue priority (s_setprio 2) changed nothing.
// bf16, P = 64 and N in {64, 128}; other cases use the general token-sequential kernel.
#include <type_traits>

#include "internal.h"

namespace ssm {
namespace {

constexpr int kVdThreads = 512;  // 256 compute + 256 staging
constexpr int kVdCompute = 256;
constexpr int kVdP = 64;
constexpr int kVdTile = 16;      // tokens per staged tile
constexpr int kVdPh = kVdP / 2;  // channels per block

// floats per staged token: B [N], C [N], a [N] (0 on a reset token), x [32], u, padding
template <int N>
constexpr int vd_row() {
    return 3 * N + kVdPh + 4;
}

// Exchange with lane i ^ 8 (DPP row_mirror, i <-> 15 - i within 16 lanes), i ^ 4 (DPP
// row_half_mirror, i <-> 7 - i within 8), i ^ 2 and i ^ 1 (DPP quad_perm): every partner
// differs from i in the named bit (and possibly lower ones), so each level halves a lane set.
template <int OFF>
__device__ __forceinline__ float vd_xchg(float v) {
    const int b = __float_as_int(v);
    int r;
    if constexpr (OFF == 8) r = __builtin_amdgcn_update_dpp(0, b, 0x140, 0xf, 0xf, false);
    else if constexpr (OFF == 4) r = __builtin_amdgcn_update_dpp(0, b, 0x141, 0xf, 0xf, false);
    else if constexpr (OFF == 2) r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xf, 0xf, false);
    else r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xf, 0xf, false);
    return __int_as_float(r);
}

// Sums of v[0..1] over the 16 lanes of a row, reduce-scatter style: at bit 3 a lane keeps
// v[bit3] and adds its partner's copy of it; bits 2, 1 and 0 add the partner's single sum.
// Lane i ends with the whole sum of index bit3(i).  Each partner agrees with the lane on
// every bit decided before and holds sums over a disjoint set of lanes.
__device__ __forceinline__ float rs16x2(const float (&v)[2], int lane) {
    const bool h8 = (lane & 8) != 0;
    float r = (h8 ? v[1] : v[0]) + vd_xchg<8>(h8 ? v[0] : v[1]);
    r += vd_xchg<4>(r);
    r += vd_xchg<2>(r);
    r += vd_xchg<1>(r);
    return r;
}

// Inclusive prefix sum over the 16 lanes of a DPP row (row_shr 1, 2, 4, 8; lanes without a
// source add 0).
__device__ __forceinline__ float vd_row_prefix(float v) {
    const int z = __float_as_int(0.0f);
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x118, 0xf, 0xf, false));
    return v;
}

// A piece's tile prefix of log a must stay within +-kVdSpan for the rescaled form (the factors
// e^{+-L} stay within 2^{+-64}, so B / P and C P keep their precision)
constexpr float kVdSpan = 44.0f;

template <int N>
__global__ void __launch_bounds__(kVdThreads) vdecay_kernel(RecurrentArgs a) {
    using D = BF16;
    using T = typename D::T;
    constexpr int R = vd_row<N>();
    constexpr int oC = N, oA = 2 * N, oX = 3 * N, oU = 3 * N + kVdPh;
    // two tile buffers: kVdTile rows of R floats, then the tile's end factors P [N] and one
    // word per 8-dimension piece (1: the piece is stored in the rescaled form)
    constexpr int kOct = N / 8;  // 8-dimension pieces per token
    constexpr int kBuf = kVdTile * R + N + kOct;
    constexpr int oP = kVdTile * R, oF = kVdTile * R + N;
    static_assert(kBuf % 4 == 0, "16-byte aligned buffers");
    __shared__ __attribute__((aligned(16))) float lds[2 * kBuf];

    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int half = blockIdx.z;  // channels 32 half .. 32 half + 31
    const int64_t g = h / (a.H / a.G);
    const int64_t ntiles = (a.T + kVdTile - 1) / kVdTile;
    const T* xs = static_cast<const T*>(a.x);
    const T* bs = static_cast<const T*>(a.Bm);
    const T* cs = static_cast<const T*>(a.Cm);

    // staging (waves 4-7): lane sl of staging wave sw handles token sl % 16 of the tile and the
    // 8-dimension piece kPPW sw + sl / 16 of B, C and the gates (so a piece's 16 tokens are the
    // 16 lanes of one DPP row), and thread sti one pair of x values, as 16-byte (B, C, gates)
    // and 4-byte (x) loads.  The loads of tile k+2 are issued right after tile k+1 is stored,
    // so they have a whole tile of compute to arrive (the registers hold one tile).
    const int sti = tid - kVdCompute;
    constexpr int kPPW = kOct / 4;  // pieces per staging wave
    const int sl = tid & 63;
    const int su_t = sl & 15, su_q = kPPW * ((sti >> 6) & 3) + (sl >> 4);
    const bool su_live = (sl >> 4) < kPPW;
    const int sx_t = sti / (kVdPh / 2), sx_p = 2 * (sti % (kVdPh / 2));  // x pair
    uint4 rb, rc;
    float4 rg0, rg1;
    bool rr;
    uint32_t rx;
    float ru;
    auto load_tile = [&](int64_t k) {
        const int64_t t0 = k * kVdTile;
        const int nt = static_cast<int>(min(static_cast<int64_t>(kVdTile), a.T - t0));
        rb = rc = make_uint4(0, 0, 0, 0);
        rg0 = rg1 = make_float4(0.f, 0.f, 0.f, 0.f);
        rr = false;
        if (su_live && su_t < nt) {
            const int64_t t = t0 + su_t;
            rb = *reinterpret_cast<const uint4*>(bs + b * a.B_sb + t * a.B_st + g * a.N + 8 * su_q);
            rc = *reinterpret_cast<const uint4*>(cs + b * a.C_sb + t * a.C_st + g * a.N + 8 * su_q);
            if (a.log_decay) {
                const float* gp = a.log_decay + ((b * a.T + t) * a.H + h) * N + 8 * su_q;
                rg0 = *reinterpret_cast<const float4*>(gp);
                rg1 = *reinterpret_cast<const float4*>(gp + 4);
            } else {
                const float d = a.dt[(b * a.T + t) * a.H + h];
                const float4 v0 = *reinterpret_cast<const float4*>(a.A_vec + h * N + 8 * su_q);
                const float4 v1 = *reinterpret_cast<const float4*>(a.A_vec + h * N + 8 * su_q + 4);
                rg0 = make_float4(d * v0.x, d * v0.y, d * v0.z, d * v0.w);
                rg1 = make_float4(d * v1.x, d * v1.y, d * v1.z, d * v1.w);
            }
            // a reset (new sequence at t) zeroes the state before token t's update, which is
            // the update with a_t = 0 (the state is finite)
            rr = a.seq_idx && t > 0 && a.seq_idx[b * a.T + t] != a.seq_idx[b * a.T + t - 1];
        }
        rx = 0u;
        if (sx_t < nt)
            rx = *reinterpret_cast<const uint32_t*>(xs + b * a.x_sb + (t0 + sx_t) * a.x_st +
                                                    h * kVdP + kVdPh * half + sx_p);
        ru = (sti < nt && a.dt) ? a.dt[(b * a.T + t0 + sti) * a.H + h] : 1.0f;
    };
    // Within a tile the compute lanes keep the state rescaled, S~_t = S_t / P_t with
    // P_t = a_1 ... a_t (per dimension, from the tile's start): then
    //     S~_t = S~_{t-1} + u_t x_t (B_t / P_t),    y_t = (C_t P_t) . S~_t,
    // two fused multiply-adds per element instead of a multiply and two, and S = P_end S~ at
    // the tile's end.  The staging lanes form L_t = log P_t (a prefix over their row), and
    // store B / P, C P and a = 1 for a piece whose L stays within +-kVdSpan on every token;
    // any other piece (a reset, a fast decay, a NaN) keeps the plain form: B, C, a_t and an end
    // factor of 1.
    auto store_tile = [&](int64_t k) {
        float* buf = lds + (k & 1) * kBuf;
        const int nt = static_cast<int>(min(static_cast<int64_t>(kVdTile), a.T - k * kVdTile));
        const bool tok = su_live && su_t < nt;
        const float lg[8] = {rg0.x, rg0.y, rg0.z, rg0.w, rg1.x, rg1.y, rg1.z, rg1.w};
        float L[8];
        bool ok = true;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // tokens past the tile's end add 0, so the row's last lane holds the end value
            L[e] = vd_row_prefix(!tok ? 0.0f : rr ? -__builtin_huge_valf() : lg[e]);
            ok = ok && L[e] >= -kVdSpan && L[e] <= kVdSpan;
        }
        const uint64_t badm = __ballot(!ok);
        const bool scaled = ((badm >> (sl & 48)) & 0xFFFFull) == 0;
        if (tok) {
            float* row = buf + su_t * R + 8 * su_q;
            const uint32_t wb[4] = {rb.x, rb.y, rb.z, rb.w}, wc[4] = {rc.x, rc.y, rc.z, rc.w};
            float fb[8], fc[8], fa[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fb[2 * e] = __uint_as_float(wb[e] << 16);
                fb[2 * e + 1] = __uint_as_float(wb[e] & 0xFFFF0000u);
                fc[2 * e] = __uint_as_float(wc[e] << 16);
                fc[2 * e + 1] = __uint_as_float(wc[e] & 0xFFFF0000u);
            }
            if (scaled) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    fb[e] *= __expf(-L[e]);
                    fc[e] *= __expf(L[e]);
                    fa[e] = 1.0f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) fa[e] = rr ? 0.0f : __expf(lg[e]);
            }
            *reinterpret_cast<float4*>(row) = make_float4(fb[0], fb[1], fb[2], fb[3]);
            *reinterpret_cast<float4*>(row + 4) = make_float4(fb[4], fb[5], fb[6], fb[7]);
            *reinterpret_cast<float4*>(row + oC) = make_float4(fc[0], fc[1], fc[2], fc[3]);
            *reinterpret_cast<float4*>(row + oC + 4) = make_float4(fc[4], fc[5], fc[6], fc[7]);
            *reinterpret_cast<float4*>(row + oA) = make_float4(fa[0], fa[1], fa[2], fa[3]);
            *reinterpret_cast<float4*>(row + oA + 4) = make_float4(fa[4], fa[5], fa[6], fa[7]);
        }
        if (su_live && su_t == kVdTile - 1) {
            // the row's last lane: the piece's end factors and its form
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = scaled ? __expf(L[e]) : 1.0f;
            *reinterpret_cast<float4*>(buf + oP + 8 * su_q) = make_float4(pe[0], pe[1], pe[2], pe[3]);
            *reinterpret_cast<float4*>(buf + oP + 8 * su_q + 4) = make_float4(pe[4], pe[5], pe[6], pe[7]);
            reinterpret_cast<uint32_t*>(buf + oF)[su_q] = scaled ? 1u : 0u;
        }
        if (sx_t < nt)
            *reinterpret_cast<float2*>(buf + sx_t * R + oX + sx_p) =
                make_float2(__uint_as_float(rx << 16), __uint_as_float(rx & 0xFFFF0000u));
        if (sti < nt) buf[sti * R + oU] = ru;
    };

    // compute lanes: channels p0, p0 + 1, dimensions n0 .. n0 + NL - 1
    constexpr int NL = N / 16;
    const int pl = 2 * (tid / 16);  // channel within the block's half
    const int p0 = kVdPh * half + pl, n0 = NL * (tid % 16);
    const bool compute = tid < kVdCompute;
    float st[2][NL];
    const int64_t sbase = ((b * a.H + h) * kVdP + p0) * N + n0;
    if (compute) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int c = 0; c < NL / 4; ++c) {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a.state_in)
                    v = *reinterpret_cast<const float4*>(a.state_in + sbase + i * N + 4 * c);
                st[i][4 * c] = v.x; st[i][4 * c + 1] = v.y;
                st[i][4 * c + 2] = v.z; st[i][4 * c + 3] = v.w;
            }
    } else {
        load_tile(0);
        store_tile(0);
        if (ntiles > 1) load_tile(1);
    }
    __syncthreads();

    T* y = static_cast<T*>(a.y);
    const int64_t y_tok = a.H * kVdP;
    // after the reduce-scatter lane tid holds channel p0 + bit3 of tid; lanes with
    // tid % 8 == 0 write it
    const int p_out = p0 + ((tid >> 3) & 1);
    T* y_p = y + (b * a.T * a.H + h) * kVdP + p_out;  // y[b, 0, h, p_out]
    // one token: decay-and-input update, per-channel read-out into acc[0..1]; TWO: every
    // piece of this wave is in the rescaled form (a = 1), so the decay multiply is left out
    auto token = [&](const float* row, float* acc, auto two) {
        constexpr bool TWO = decltype(two)::value;
        const float u = row[oU];
        const float2 x2 = *reinterpret_cast<const float2*>(row + oX + pl);
        const float dx[2] = {u * x2.x, u * x2.y};
        float bv[NL], av[NL], cv[NL];
#pragma unroll
        for (int c = 0; c < NL / 4; ++c) {
            const float4 b4 = *reinterpret_cast<const float4*>(row + n0 + 4 * c);
            const float4 c4 = *reinterpret_cast<const float4*>(row + oC + n0 + 4 * c);
            bv[4 * c] = b4.x; bv[4 * c + 1] = b4.y; bv[4 * c + 2] = b4.z; bv[4 * c + 3] = b4.w;
            cv[4 * c] = c4.x; cv[4 * c + 1] = c4.y; cv[4 * c + 2] = c4.z; cv[4 * c + 3] = c4.w;
            if (!TWO) {
                const float4 a4 = *reinterpret_cast<const float4*>(row + oA + n0 + 4 * c);
                av[4 * c] = a4.x; av[4 * c + 1] = a4.y; av[4 * c + 2] = a4.z; av[4 * c + 3] = a4.w;
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float s_ = 0.0f;
#pragma unroll
            for (int e = 0; e < NL; ++e) {
                // both steps update the state register in place (a multiply, then an
                // accumulate), so the loop carries no register copies
                if (!TWO) st[i][e] *= av[e];
                st[i][e] = __builtin_fmaf(dx[i], bv[e], st[i][e]);
                s_ = __builtin_fmaf(cv[e], st[i][e], s_);
            }
            acc[i] = s_;
        }
    };
    // a tile's tokens; the reduce-scatter of a token runs in the next token's iteration
    auto tile_tokens = [&](const float* buf, int64_t t0, int nt, auto two) {
        float pend[2] = {0.0f, 0.0f};
#pragma unroll 4
        for (int tt = 0; tt < nt; ++tt) {
            float acc[2];
            token(buf + tt * R, acc, two);
            if (tt > 0) {
                const float yv = rs16x2(pend, tid);
                if ((tid & 7) == 0) D::store(y_p, (t0 + tt - 1) * y_tok, yv);
            }
            pend[0] = acc[0];
            pend[1] = acc[1];
        }
        if (nt > 0) {
            const float yv = rs16x2(pend, tid);
            if ((tid & 7) == 0) D::store(y_p, (t0 + nt - 1) * y_tok, yv);
        }
    };
    for (int64_t k = 0; k < ntiles; ++k) {
        if (compute) {
            const float* buf = lds + (k & 1) * kBuf;
            const int64_t t0 = k * kVdTile;
            const int nt = static_cast<int>(min(static_cast<int64_t>(kVdTile), a.T - t0));
            const bool lane_scaled = reinterpret_cast<const uint32_t*>(buf + oF)[n0 / 8] != 0;
            if (__ballot(!lane_scaled) == 0)
                tile_tokens(buf, t0, nt, std::true_type{});
            else
                tile_tokens(buf, t0, nt, std::false_type{});
            // back from the rescaled state (end factor 1 for a piece in the plain form)
#pragma unroll
            for (int c = 0; c < NL / 4; ++c) {
                const float4 p4 = *reinterpret_cast<const float4*>(buf + oP + n0 + 4 * c);
                const float pe[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[i][4 * c + e] *= pe[e];
            }
        } else if (k + 1 < ntiles) {
            store_tile(k + 1);  // the other buffer, last read before the previous barrier
            if (k + 2 < ntiles) load_tile(k + 2);
        }
        __syncthreads();
    }
    if (compute && a.state_out) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int c = 0; c < NL / 4; ++c)
                *reinterpret_cast<float4*>(a.state_out + sbase + i * N + 4 * c) =
                    make_float4(st[i][4 * c], st[i][4 * c + 1], st[i][4 * c + 2], st[i][4 * c + 3]);
    }
}

}  // namespace

bool vdecay_supported(int64_t P, int64_t N) { return P == kVdP && (N == 64 || N == 128); }

// bf16 rows with 16-byte aligned, contiguous B / C / gate pieces take vdecay_kernel; anything
// else the general token-sequential kernel's vector mode
hipError_t launch_vdecay(const RecurrentArgs& a, ssm_dtype_t dtype, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (vchunk_supported(a, dtype)) return launch_vchunk(a, stream);
    const uintptr_t al = reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.Bm) |
                         reinterpret_cast<uintptr_t>(a.Cm) | reinterpret_cast<uintptr_t>(a.log_decay) |
                         reinterpret_cast<uintptr_t>(a.A_vec);
    const bool fast = dtype == SSM_BF16 && vdecay_supported(a.P, a.N) && (al & 15) == 0 &&
                      a.x_sc == 1 && a.B_sc == 1 && a.C_sc == 1 && a.B_st % 8 == 0 &&
                      a.C_st % 8 == 0 && a.B_sb % 8 == 0 && a.C_sb % 8 == 0 &&
                      a.x_st % 2 == 0 && a.x_sb % 2 == 0;
    if (!fast) return launch_recurrent(a, dtype, stream);
    dim3 grid(static_cast<unsigned>(a.H), static_cast<unsigned>(a.B), 2);  // z: channel half
    if (a.N == 128)
        vdecay_kernel<128><<<grid, kVdThreads, 0, stream>>>(a);
    else
        vdecay_kernel<64><<<grid, kVdThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace ssm
