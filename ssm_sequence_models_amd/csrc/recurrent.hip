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
// The N/4 lanes that share a channel p are adjacent, so y[p] is a butterfly reduction over
// that lane group.
#include "internal.h"

namespace ssm {
namespace {

template <class D, int J>
__global__ void __launch_bounds__(256)
recurrent_kernel(RecurrentArgs a, int nthreads) {
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
            const float4 v = *reinterpret_cast<const float4*>(a.state_in + base + e);
            st[j][0] = v.x; st[j][1] = v.y; st[j][2] = v.z; st[j][3] = v.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) st[j][k] = 0.0f;
        }
    }

    const T* xs = static_cast<const T*>(a.x);
    const T* bs = static_cast<const T*>(a.Bm);
    const T* cs = static_cast<const T*>(a.Cm);
    const float Ah = a.A[h];
    for (int64_t t = 0; t < a.T; ++t) {
        if (a.seq_idx && t > 0 && a.seq_idx[b * a.T + t] != a.seq_idx[b * a.T + t - 1]) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k) st[j][k] = 0.0f;
        }
        const float d = a.dt[(b * a.T + t) * a.H + h];
        const float dec = __expf(d * Ah);
        float Bv[4], Cv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t n = n0 + k;
            Bv[k] = active ? D::load(bs, b * a.B_sb + t * a.B_st + (g * a.N + n) * a.B_sc) : 0.0f;
            Cv[k] = active ? D::load(cs, b * a.C_sb + t * a.C_st + (g * a.N + n) * a.C_sc) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t e = static_cast<int64_t>(j) * 4 * nthreads + 4 * tid;
            const bool live = active && e < PN;
            const int64_t p = live ? e / a.N : 0;
            const float xp = live ? D::load(xs, b * a.x_sb + t * a.x_st + (h * a.P + p) * a.x_sc) : 0.0f;
            const float dx = d * xp;
            float part = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                st[j][k] = __builtin_fmaf(dec, st[j][k], dx * Bv[k]);
                part = __builtin_fmaf(Cv[k], st[j][k], part);
            }
            for (int off = lanes_per_p / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
            if (live && n0 == 0) D::store(y, ((b * a.T + t) * a.H + h) * a.P + p, part);
        }
    }
    if (a.state_out) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t e = static_cast<int64_t>(j) * 4 * nthreads + 4 * tid;
            if (active && e < PN)
                *reinterpret_cast<float4*>(a.state_out + base + e) =
                    make_float4(st[j][0], st[j][1], st[j][2], st[j][3]);
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
// per thread at 256 threads.
bool recurrent_supported(int64_t P, int64_t N) {
    if (N % 4 != 0) return false;
    const int64_t lp = N / 4;
    if (lp > 64 || (lp & (lp - 1)) != 0) return false;
    return P * N <= 256 * 4 * 16;
}

hipError_t launch_recurrent(const RecurrentArgs& a, ssm_dtype_t dtype, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    const int64_t PN = a.P * a.N;
    int64_t nthreads = PN / 4;
    if (nthreads > 256) nthreads = 256;
    // whole lane groups per thread run, and a block of whole wavefronts
    const int block = static_cast<int>(((nthreads + 63) / 64) * 64);
    const int64_t runs = (PN + 4 * nthreads - 1) / (4 * nthreads);
    dim3 grid(a.H, a.B);
    const int nt = static_cast<int>(nthreads);
#define SSM_REC(JJ)                                                                         \
    if (runs <= JJ) {                                                                       \
        if (dtype == SSM_BF16)                                                              \
            recurrent_kernel<BF16, JJ><<<grid, block, 0, stream>>>(a, nt);                  \
        else                                                                                \
            recurrent_kernel<F32, JJ><<<grid, block, 0, stream>>>(a, nt);                   \
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
