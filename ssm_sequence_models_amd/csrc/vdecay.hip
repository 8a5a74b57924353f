// vdecay.hip -- the scan with a diagonal transition (one decay per state dimension) for long
// rows: length-generalization reading notes, Sec. 2.1 Eq. (1) with A_t = diag(a_t) and
// Sec. 2.5's diagonal case (the transition taken from log coefficients), per head h, channel
// p and state dimension n:
//     state[p][n] <- a_t[n] state[p][n] + u_t x_t[p] B_t[n],    y_t[p] = C_t . state[p][:]
// with log a_t[n] = log_decay[b][t][h][n] or dt_t A_vec[h][n], u_t = dt_t (or 1).
//
// Token-sequential, laid out for issue rate rather than for the decode step's one token:
//   - one block per (row, head), 512 threads: waves 0-3 compute, waves 4-7 stage;
//   - a compute lane owns a 4 x NL block of the state (channels p = 4 (tid / 16) .. +3,
//     dimensions n = NL (tid % 16) .. +NL-1, NL = N / 16) in registers for the whole row.
//     Per token it reads its NL values of B, C and a_t and its 4 values of x from LDS (lanes
//     sharing them read the same addresses), issues 4 NL independent decay-and-input updates
//     and 4 NL read-out products, and a reduce-scatter over the 16 lanes of its channel block
//     leaves y_t[p] of one channel in every fourth lane.  A quarter-row-per-lane layout spent
//     its time returning LDS data (24 16-byte reads per token and lane; 4.6 ms against 4.1 ms
//     at the 1.3B-like shape); pairing tokens under one reduce-scatter raised the register
//     count to 139 and ran slower (5.5 ms).  Each token's reduce-scatter runs in the next
//     token's iteration, where nothing depends on it, so its exchange latency overlaps that
//     token's updates.  Letting all eight waves compute (4 x 4 blocks, a 32-lane reduction
//     through ds_swizzle, tiles prefetched into registers) ran slower too (3.65-3.80 ms
//     against 3.3 ms);
//   - the staging waves copy a tile of 32 tokens (B, C, x, dt, and a_t[n] = exp(log a_t[n]),
//     formed here once per token and dimension; a_t = 0 where seq_idx starts a new sequence,
//     which is the reset) into one of two LDS
//     buffers while the compute waves consume the other: one barrier per tile, global
//     latency hidden behind the previous tile's arithmetic.
// P = 64 and N in {64, 128}; other shapes use the general token-sequential kernel.
#include "internal.h"

namespace ssm {
namespace {

constexpr int kVdThreads = 512;  // 256 compute + 256 staging
constexpr int kVdCompute = 256;
constexpr int kVdP = 64;
constexpr int kVdTile = 32;      // tokens per staged tile

// floats per staged token: B [N], C [N], a [N] (0 on a reset token), x [64], u, padding
template <int N>
constexpr int vd_row() {
    return 3 * N + kVdP + 4;
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

// Sums of v[0..3] over the 16 lanes of a row, reduce-scatter style: at the bit-3 level a lane
// keeps the pair {0, 1} (bit clear) or {2, 3} (bit set) and adds its partner's copy of that
// pair; at bit 2 it keeps one of the two; bits 1 and 0 add the partner's single sum.  Lane i
// ends with the whole sum of index 2 bit3(i) + bit2(i).  Each partner agrees with the lane on
// every bit decided before and holds sums over a disjoint set of lanes.
__device__ __forceinline__ float rs16x4(const float (&v)[4], int lane) {
    const bool h8 = (lane & 8) != 0, h4 = (lane & 4) != 0;
    const float k0 = h8 ? v[2] : v[0], k1 = h8 ? v[3] : v[1];
    const float s0 = h8 ? v[0] : v[2], s1 = h8 ? v[1] : v[3];
    const float w0 = k0 + vd_xchg<8>(s0), w1 = k1 + vd_xchg<8>(s1);
    const float keep = h4 ? w1 : w0, send = h4 ? w0 : w1;
    float r = keep + vd_xchg<4>(send);
    r += vd_xchg<2>(r);
    r += vd_xchg<1>(r);
    return r;
}

template <class D, int N>
__global__ void __launch_bounds__(kVdThreads) vdecay_kernel(RecurrentArgs a) {
    using T = typename D::T;
    constexpr int R = vd_row<N>();
    constexpr int oC = N, oA = 2 * N, oX = 3 * N, oU = 3 * N + kVdP;
    __shared__ __attribute__((aligned(16))) float lds[2 * kVdTile * R];  // two tile buffers

    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int64_t g = h / (a.H / a.G);
    const int64_t ntiles = (a.T + kVdTile - 1) / kVdTile;
    const T* xs = static_cast<const T*>(a.x);
    const T* bs = static_cast<const T*>(a.Bm);
    const T* cs = static_cast<const T*>(a.Cm);

    // staging: tile k of tokens into buffer k & 1 (staging waves only).  Every load of the
    // tile is issued before the first LDS store (the loops have compile-time trip counts), so
    // the tile costs about one global latency rather than one per element.
    auto stage = [&](int64_t k) {
        constexpr int kItems = kVdTile * N / kVdCompute;   // B / C / gate values per thread
        constexpr int kXItems = kVdTile * kVdP / kVdCompute;
        const int st = tid - kVdCompute;
        float* buf = lds + (k & 1) * (kVdTile * R);
        const int64_t t0 = k * kVdTile;
        const int nt = static_cast<int>(min(static_cast<int64_t>(kVdTile), a.T - t0));
        float vb[kItems], vc[kItems], vg[kItems], vx[kXItems];
        bool rs[kItems];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const int i = st + j * kVdCompute;
            const int tt = i / N, n = i % N;
            const int64_t t = t0 + tt;
            vb[j] = vc[j] = vg[j] = 0.0f;
            rs[j] = false;
            if (tt < nt) {
                vb[j] = D::load(bs, b * a.B_sb + t * a.B_st + (g * a.N + n) * a.B_sc);
                vc[j] = D::load(cs, b * a.C_sb + t * a.C_st + (g * a.N + n) * a.C_sc);
                vg[j] = a.log_decay ? a.log_decay[((b * a.T + t) * a.H + h) * N + n]
                                    : a.dt[(b * a.T + t) * a.H + h] * a.A_vec[h * N + n];
                // a reset (new sequence at t) zeroes the state before token t's update, which
                // is the update with a_t = 0 (the state is finite)
                rs[j] = a.seq_idx && t > 0 && a.seq_idx[b * a.T + t] != a.seq_idx[b * a.T + t - 1];
            }
        }
#pragma unroll
        for (int j = 0; j < kXItems; ++j) {
            const int i = st + j * kVdCompute;
            const int tt = i / kVdP, p = i % kVdP;
            vx[j] = tt < nt ? D::load(xs, b * a.x_sb + (t0 + tt) * a.x_st + (h * kVdP + p) * a.x_sc)
                            : 0.0f;
        }
        float vu = 1.0f;
        if (st < nt && a.dt) vu = a.dt[(b * a.T + t0 + st) * a.H + h];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const int i = st + j * kVdCompute;
            const int tt = i / N, n = i % N;
            if (tt < nt) {
                float* row = buf + tt * R;
                row[n] = vb[j];
                row[oC + n] = vc[j];
                row[oA + n] = rs[j] ? 0.0f : __expf(vg[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kXItems; ++j) {
            const int i = st + j * kVdCompute;
            const int tt = i / kVdP, p = i % kVdP;
            if (tt < nt) buf[tt * R + oX + p] = vx[j];
        }
        if (st < nt) buf[st * R + oU] = vu;
    };

    // compute lanes: channels p0 .. p0 + 3, dimensions n0 .. n0 + NL - 1
    constexpr int NL = N / 16;
    const int p0 = 4 * (tid / 16), n0 = NL * (tid % 16);
    const bool compute = tid < kVdCompute;
    float st[4][NL];
    const int64_t sbase = ((b * a.H + h) * kVdP + p0) * N + n0;
    if (compute) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < NL / 4; ++c) {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a.state_in)
                    v = *reinterpret_cast<const float4*>(a.state_in + sbase + i * N + 4 * c);
                st[i][4 * c] = v.x; st[i][4 * c + 1] = v.y;
                st[i][4 * c + 2] = v.z; st[i][4 * c + 3] = v.w;
            }
    } else {
        stage(0);
    }
    __syncthreads();

    T* y = static_cast<T*>(a.y);
    const int64_t y_tok = a.H * kVdP;
    // after the reduce-scatter lane tid holds channel p0 + 2 bit3 + bit2 of tid; lanes with
    // tid % 4 == 0 write it
    const int p_out = p0 + ((tid >> 2) & 3);
    T* y_p = y + (b * a.T * a.H + h) * kVdP + p_out;  // y[b, 0, h, p_out]
    // one token: reset if flagged, decay-and-input update, per-channel read-out into acc[0..3]
    auto token = [&](const float* row, float* acc) {
        const float u = row[oU];
        const float4 x4 = *reinterpret_cast<const float4*>(row + oX + p0);
        const float dx[4] = {u * x4.x, u * x4.y, u * x4.z, u * x4.w};
        float bv[NL], av[NL], cv[NL];
#pragma unroll
        for (int c = 0; c < NL / 4; ++c) {
            const float4 b4 = *reinterpret_cast<const float4*>(row + n0 + 4 * c);
            const float4 a4 = *reinterpret_cast<const float4*>(row + oA + n0 + 4 * c);
            const float4 c4 = *reinterpret_cast<const float4*>(row + oC + n0 + 4 * c);
            bv[4 * c] = b4.x; bv[4 * c + 1] = b4.y; bv[4 * c + 2] = b4.z; bv[4 * c + 3] = b4.w;
            av[4 * c] = a4.x; av[4 * c + 1] = a4.y; av[4 * c + 2] = a4.z; av[4 * c + 3] = a4.w;
            cv[4 * c] = c4.x; cv[4 * c + 1] = c4.y; cv[4 * c + 2] = c4.z; cv[4 * c + 3] = c4.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s_ = 0.0f;
#pragma unroll
            for (int e = 0; e < NL; ++e) {
                // both steps update the state register in place (a multiply, then an
                // accumulate), so the loop carries no register copies
                st[i][e] *= av[e];
                st[i][e] = __builtin_fmaf(dx[i], bv[e], st[i][e]);
                s_ = __builtin_fmaf(cv[e], st[i][e], s_);
            }
            acc[i] = s_;
        }
    };
    for (int64_t k = 0; k < ntiles; ++k) {
        if (compute) {
            const float* buf = lds + (k & 1) * (kVdTile * R);
            const int64_t t0 = k * kVdTile;
            const int nt = static_cast<int>(min(static_cast<int64_t>(kVdTile), a.T - t0));
            // software pipeline: token tt's reduction runs in the next iteration, where
            // nothing it computes depends on it, so its exchange latency overlaps token
            // tt + 1's updates
            float pend[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int tt = 0; tt < nt; ++tt) {
                float acc[4];
                token(buf + tt * R, acc);
                if (tt > 0) {
                    const float yv = rs16x4(pend, tid);
                    if ((tid & 3) == 0) D::store(y_p, (t0 + tt - 1) * y_tok, yv);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) pend[i] = acc[i];
            }
            if (nt > 0) {
                const float yv = rs16x4(pend, tid);
                if ((tid & 3) == 0) D::store(y_p, (t0 + nt - 1) * y_tok, yv);
            }
        } else if (k + 1 < ntiles) {
            stage(k + 1);
        }
        __syncthreads();
    }
    if (compute && a.state_out) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < NL / 4; ++c)
                *reinterpret_cast<float4*>(a.state_out + sbase + i * N + 4 * c) =
                    make_float4(st[i][4 * c], st[i][4 * c + 1], st[i][4 * c + 2], st[i][4 * c + 3]);
    }
}

}  // namespace

bool vdecay_supported(int64_t P, int64_t N) { return P == kVdP && (N == 64 || N == 128); }

hipError_t launch_vdecay(const RecurrentArgs& a, ssm_dtype_t dtype, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    if (a.N == 128) {
        if (dtype == SSM_BF16)
            vdecay_kernel<BF16, 128><<<grid, kVdThreads, 0, stream>>>(a);
        else
            vdecay_kernel<F32, 128><<<grid, kVdThreads, 0, stream>>>(a);
    } else {
        if (dtype == SSM_BF16)
            vdecay_kernel<BF16, 64><<<grid, kVdThreads, 0, stream>>>(a);
        else
            vdecay_kernel<F32, 64><<<grid, kVdThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace ssm
