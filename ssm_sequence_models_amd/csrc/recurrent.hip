// recurrent.hip -- token-sequential form of the selective scan: the decode step on a state
// pool, and the scan path for shapes / dtypes the chunked MFMA kernel does not take.
//
// Length-generalization reading notes, Sec. 2.1 Eq. (1), per head h and channel p:
//     state[p,:] <- exp(dt_t A_h) state[p,:] + dt_t x_t[p] B_t,     y_t[p] = C_t . state[p,:]
// starting from the given initial state (Sec. 2.5 / 2.6) and, on packed rows, from zero
// where seq_idx changes.
//
// One block per (row, head).  The fp32 state [P, N] stays in registers for the whole token
// loop: thread `tid` owns the float4 runs e = j*4*NT + 4*tid .. +3 (row-major over [P, N]),
// which makes the one read and one write of the state fully coalesced 16-byte accesses --
// for the decode step the state traffic (2 x 32 KiB per request and head) is the whole cost.
// The N/4 lanes that share a channel p are adjacent, so y[p] is a reduction over that lane
// group.  When the runs tile the state exactly and N = 128 (32 lanes per channel; P = 64 gives
// 4 runs of 2048 values at 512 threads), the J sums of a lane are reduced together,
// reduce-scatter style: at each halving of the lane span a lane keeps half of its sums and
// adds its partner's matching half, so J = 4 sums over 32 lanes take 2 + 1 exchanges and three
// more for the last 8 lanes (6 instead of 20).
// The token loop reads its inputs from LDS: tiles of up to 16 tokens of B, C, x and dt
// (and the sequence resets) are staged by the whole block with loads ordered along the
// contiguous dimension, so a token costs no memory round trip and the first tile's loads
// overlap the state load.
// VEC: the diagonal transition of Eq. (1) (A_t = diag(a_t), one decay per state dimension,
// Sec. 2.5's diagonal case): the tile also holds a_t[n] = exp(log a_t[n]) for every n,
// computed once per token by the staging threads, and each state element takes its own
// dimension's decay; dt may be absent (= 1).
#include "internal.h"

namespace ssm {
namespace {

// Exchange with the partner lane of level `off` inside a 32-lane group: off 16 pairs lane i
// with i ^ 16 (ds_swizzle), off 8 with i ^ 15 (DPP row_mirror), off 4 with i ^ 7 (DPP
// row_half_mirror), off 2 and 1 with i ^ 2 and i ^ 1 (DPP quad_perm).  Each partner differs
// from i in the bit `off`, and together the five relations reach all 32 lanes.
template <int OFF>
__device__ __forceinline__ float xchg(float v) {
    const int b = __float_as_int(v);
    int r;
    if constexpr (OFF == 16) r = __builtin_amdgcn_ds_swizzle(b, 0x401F);  // and 0x1f, xor 0x10
    else if constexpr (OFF == 8) r = __builtin_amdgcn_update_dpp(0, b, 0x140, 0xf, 0xf, false);
    else if constexpr (OFF == 4) r = __builtin_amdgcn_update_dpp(0, b, 0x141, 0xf, 0xf, false);
    else if constexpr (OFF == 2) r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xf, 0xf, false);
    else r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xf, 0xf, false);
    return __int_as_float(r);
}

// One level of the reduce-scatter over the J sums: a lane keeps the half of its `cnt` sums
// chosen by bit OFF of its lane index and adds its partner's copy of that half; once one sum
// is left, levels add the partner's sum.  The partner holds the same index set (it agrees with
// the lane on every bit decided so far) and sums over a disjoint set of lanes.
template <int J, int OFF>
__device__ __forceinline__ void rs_level(float (&v)[J], int& cnt, int& j_off, int lane) {
    if (cnt > 1) {
        const bool hi = (lane & OFF) != 0;
        const int half = cnt / 2;
#pragma unroll
        for (int i = 0; i < J / 2; ++i) {
            if (i < half) {
                const float send = hi ? v[i] : v[i + half];
                const float mine = hi ? v[i + half] : v[i];
                v[i] = mine + xchg<OFF>(send);
            }
        }
        j_off += hi ? half : 0;
        cnt = half;
    } else {
        v[0] += xchg<OFF>(v[0]);
    }
}

// Sum over the 32 adjacent lanes sharing each of the J channels v[j] belongs to.  Returns the
// sum for channel index *jr (the lane's reduce-scatter position); the lanes with
// lane % (32 / J) == 0 are the writers (see the caller).
template <int J>
__device__ __forceinline__ float reduce_scatter32(float (&v)[J], int lane, int* jr) {
    int j_off = 0, cnt = J;
    rs_level<J, 16>(v, cnt, j_off, lane);
    rs_level<J, 8>(v, cnt, j_off, lane);
    rs_level<J, 4>(v, cnt, j_off, lane);
    rs_level<J, 2>(v, cnt, j_off, lane);
    rs_level<J, 1>(v, cnt, j_off, lane);
    *jr = j_off;
    return v[0];
}

constexpr int kTileTMax = 16;
constexpr size_t kTileBytesMax = 48 * 1024;

// Stage the [nt][cnt] tile, element (tt, r) at src[base + (t0 + tt) s_t + r s_c], into
// dst[tt * row + r] (floats); consecutive threads take consecutive addresses of whichever
// index has the smaller stride.
template <class D>
__device__ __forceinline__ void stage_tile(const typename D::T* src, int64_t base, int64_t t0,
                                           int64_t s_t, int64_t s_c, int nt, int cnt,
                                           float* dst, int row) {
    const int n = nt * cnt;
    if (s_t < s_c) {
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int tt = i % nt, r = i / nt;
            dst[tt * row + r] = D::load(src, base + (t0 + tt) * s_t + r * s_c);
        }
    } else {
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int r = i % cnt, tt = i / cnt;
            dst[tt * row + r] = D::load(src, base + (t0 + tt) * s_t + r * s_c);
        }
    }
}

constexpr int kRecThreads = 512;

template <class D, int J, bool VEC>
__global__ void __launch_bounds__(kRecThreads)
recurrent_kernel(RecurrentArgs a, int nthreads, int tile_t) {
    using T = typename D::T;
    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t PN = a.P * a.N;
    const int lanes_per_p = static_cast<int>(a.N / 4);
    const int64_t g = h / (a.H / a.G);
    T* y = static_cast<T*>(a.y);

    const int64_t slot = a.indices ? static_cast<int64_t>(a.indices[b]) : b;
    if (slot < 0 || slot >= a.n_slots) {
        // skipped row: zero its outputs, leave the state alone
        for (int64_t i = tid; i < a.T * a.P; i += blockDim.x) {
            const int64_t t = i / a.P, p = i % a.P;
            D::store(y, ((b * a.T + t) * a.H + h) * a.P + p, 0.0f);
        }
        return;
    }
    const bool active = tid < nthreads;
    const int64_t base = (slot * a.H + h) * PN;
    const int n0 = (tid * 4) % static_cast<int>(a.N);

    float st[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t e = static_cast<int64_t>(j) * 4 * nthreads + 4 * tid;
        if (active && e < PN && a.state_in) {
            // the state is read once and written once: non-temporal accesses (they keep it
            // out of the caches' way and measured faster on a plain 1 GiB read-modify-write)
            const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.state_in + base + e));
            st[j][0] = v[0]; st[j][1] = v[1]; st[j][2] = v[2]; st[j][3] = v[3];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) st[j][k] = 0.0f;
        }
    }

    const T* xs = static_cast<const T*>(a.x);
    const T* bs = static_cast<const T*>(a.Bm);
    const T* cs = static_cast<const T*>(a.Cm);
    const float Ah = VEC ? 0.0f : a.A[h];
    // per staged token: B [N], C [N], (with VEC the decays [N]), x [P], dt, reset flag, padded
    // to whole 16-byte units so the per-lane B / C / decay quadruples are single LDS reads
    extern __shared__ float4 s_in4[];
    float* s_in = reinterpret_cast<float*>(s_in4);
    const int N = static_cast<int>(a.N), P = static_cast<int>(a.P);
    const int oD = 2 * N, oX = VEC ? 3 * N : 2 * N, oDt = oX + P, oF = oDt + 1;
    const int row = (oF + 1 + 3) & ~3;
    // per run: its channel p (or -1 when the run is past the state), fixed for the whole loop
    int p_of[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t e = static_cast<int64_t>(j) * 4 * nthreads + 4 * tid;
        p_of[j] = (active && e < PN) ? static_cast<int>(e / a.N) : -1;
    }
    const bool rs_path = J <= 32 && lanes_per_p == 32 && PN == static_cast<int64_t>(J) * 4 * nthreads;
    T* y_bh = y + (b * a.T * a.H + h) * a.P;  // y[b, 0, h, 0]; token t adds t * H * P
    const int64_t y_tok = a.H * a.P;
    for (int64_t tb = 0; tb < a.T; tb += tile_t) {
        const int nt = static_cast<int>(min(static_cast<int64_t>(tile_t), a.T - tb));
        __syncthreads();  // the previous tile has been consumed
        stage_tile<D>(bs, b * a.B_sb + g * a.N * a.B_sc, tb, a.B_st, a.B_sc, nt, N, s_in, row);
        stage_tile<D>(cs, b * a.C_sb + g * a.N * a.C_sc, tb, a.C_st, a.C_sc, nt, N, s_in + N, row);
        stage_tile<D>(xs, b * a.x_sb + h * a.P * a.x_sc, tb, a.x_st, a.x_sc, nt, P, s_in + oX, row);
        if constexpr (VEC) {
            // a_t[n], consecutive threads on consecutive n (the contiguous index of log_decay)
            for (int i = threadIdx.x; i < nt * N; i += blockDim.x) {
                const int tt = i / N, n = i % N;
                const int64_t t = tb + tt;
                const float lg = a.log_decay
                                     ? a.log_decay[((b * a.T + t) * a.H + h) * a.N + n]
                                     : a.dt[(b * a.T + t) * a.H + h] * a.A_vec[h * a.N + n];
                s_in[tt * row + oD + n] = __expf(lg);
            }
        }
        for (int tt = threadIdx.x; tt < nt; tt += blockDim.x) {
            const int64_t t = tb + tt;
            s_in[tt * row + oDt] = a.dt ? a.dt[(b * a.T + t) * a.H + h] : 1.0f;
            const bool reset = a.seq_idx && t > 0 && a.seq_idx[b * a.T + t] != a.seq_idx[b * a.T + t - 1];
            s_in[tt * row + oF] = reset ? 1.0f : 0.0f;
        }
        __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
        const int64_t t = tb + tt;
        const float* tin = s_in + tt * row;
        if (tin[oF] != 0.0f) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k) st[j][k] = 0.0f;
        }
        const float d = tin[oDt];
        // row % 4 == 0 and n0 % 4 == 0: 16-byte aligned quadruples
        const float4 b4 = active ? *reinterpret_cast<const float4*>(tin + n0) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 c4 = active ? *reinterpret_cast<const float4*>(tin + N + n0) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float Bv[4] = {b4.x, b4.y, b4.z, b4.w};
        const float Cv[4] = {c4.x, c4.y, c4.z, c4.w};
        float dec[4];
        if constexpr (VEC) {
            const float4 d4 = active ? *reinterpret_cast<const float4*>(tin + oD + n0) : make_float4(0.f, 0.f, 0.f, 0.f);
            dec[0] = d4.x; dec[1] = d4.y; dec[2] = d4.z; dec[3] = d4.w;
        } else {
            const float dsc = __expf(d * Ah);
#pragma unroll
            for (int k = 0; k < 4; ++k) dec[k] = dsc;
        }
        float part[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const float xp = p_of[j] >= 0 ? tin[oX + p_of[j]] : 0.0f;
            const float dx = d * xp;
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                st[j][k] = __builtin_fmaf(dec[k], st[j][k], dx * Bv[k]);
                acc = __builtin_fmaf(Cv[k], st[j][k], acc);
            }
            part[j] = acc;
        }
        T* y_t = y_bh + t * y_tok;
        if (rs_path) {
            // run j of thread tid is channel p = (4 nthreads / N) j + tid / 32; lanes tid % 32
            // share it; after the reduce-scatter the lanes with tid % (32 / J) == 0 hold whole sums
            int jr;
            const float yv = reduce_scatter32<J>(part, tid, &jr);
            if ((tid & (32 / J - 1)) == 0)
                D::store(y_t, (4 * nthreads / 128) * jr + tid / 32, yv);
        } else {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                float v = part[j];
                for (int off = lanes_per_p / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
                if (p_of[j] >= 0 && n0 == 0) D::store(y_t, p_of[j], v);
            }
        }
    }
    }
    if (a.state_out) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t e = static_cast<int64_t>(j) * 4 * nthreads + 4 * tid;
            if (active && e < PN)
                __builtin_nontemporal_store(f32x4_t{st[j][0], st[j][1], st[j][2], st[j][3]},
                                            reinterpret_cast<f32x4_t*>(a.state_out + base + e));
        }
    }
}

__global__ void copy_or_zero_f32_kernel(float* dst, const float* src, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}
__global__ void copy_or_zero_u8_kernel(uint8_t* dst, const uint8_t* src, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0;
}

}  // namespace

// Lane groups of N/4 must be a power of two within one wavefront; P*N up to 16 float4 runs
// per thread at kRecThreads threads.
bool recurrent_supported(int64_t P, int64_t N, bool vector_decay) {
    if (N % 4 != 0) return false;
    const int64_t lp = N / 4;
    if (lp > 64 || (lp & (lp - 1)) != 0) return false;
    // one staged token (B, C, x, dt, flag, and the decays) must fit the tile budget
    const int64_t row = ((vector_decay ? 3 * N : 2 * N) + P + 2 + 3) / 4 * 4;
    return P * N <= kRecThreads * 4 * 16 && row * 4 <= static_cast<int64_t>(kTileBytesMax);
}

hipError_t launch_recurrent(const RecurrentArgs& a, ssm_dtype_t dtype, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    const int64_t PN = a.P * a.N;
    int64_t nthreads = PN / 4;
    if (nthreads > kRecThreads) nthreads = kRecThreads;
    // whole lane groups per thread run, and a block of whole wavefronts
    const int block = static_cast<int>(((nthreads + 63) / 64) * 64);
    const int64_t runs = (PN + 4 * nthreads - 1) / (4 * nthreads);
    dim3 grid(a.H, a.B);
    const int nt = static_cast<int>(nthreads);
    // tokens per staged tile: up to kTileTMax, within kTileBytesMax of LDS
    const bool vec = a.log_decay != nullptr || a.A_vec != nullptr;
    // the kernel's padded token row: (B, C, [decays,] x, dt, flag) rounded up to 4 floats
    const size_t row_bytes =
        static_cast<size_t>(((vec ? 3 : 2) * a.N + a.P + 2 + 3) / 4 * 4) * sizeof(float);
    int tile_t = static_cast<int>(kTileBytesMax / row_bytes);
    if (tile_t > kTileTMax) tile_t = kTileTMax;
    if (tile_t < 1) return hipErrorInvalidValue;  // excluded by recurrent_supported
    const size_t lds = static_cast<size_t>(tile_t) * row_bytes;
#define SSM_REC(JJ)                                                                         \
    if (runs <= JJ) {                                                                       \
        if (dtype == SSM_BF16 && vec)                                                       \
            recurrent_kernel<BF16, JJ, true><<<grid, block, lds, stream>>>(a, nt, tile_t);  \
        else if (dtype == SSM_BF16)                                                         \
            recurrent_kernel<BF16, JJ, false><<<grid, block, lds, stream>>>(a, nt, tile_t); \
        else if (vec)                                                                       \
            recurrent_kernel<F32, JJ, true><<<grid, block, lds, stream>>>(a, nt, tile_t);   \
        else                                                                                \
            recurrent_kernel<F32, JJ, false><<<grid, block, lds, stream>>>(a, nt, tile_t);  \
        return hipGetLastError();                                                           \
    }
    SSM_REC(1) SSM_REC(2) SSM_REC(4) SSM_REC(8) SSM_REC(16)
#undef SSM_REC
    return hipErrorInvalidValue;
}

hipError_t launch_copy_or_zero_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
    if (n == 0 || dst == nullptr || dst == src) return hipSuccess;
    copy_or_zero_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(dst, src, n);
    return hipGetLastError();
}

hipError_t launch_copy_or_zero_bytes(void* dst, const void* src, int64_t nbytes, hipStream_t s) {
    if (nbytes == 0 || dst == nullptr || dst == src) return hipSuccess;
    copy_or_zero_u8_kernel<<<static_cast<unsigned>((nbytes + 255) / 256), 256, 0, s>>>(
        static_cast<uint8_t*>(dst), static_cast<const uint8_t*>(src), nbytes);
    return hipGetLastError();
}

}  // namespace ssm
