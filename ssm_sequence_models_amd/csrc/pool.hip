// pool.hip -- the prefill reading its initial states from, and writing its final states to,
// the decode pools (causal-conv1d tutorial, ch. 7: "the physical cache may exceed the minimal
// history" (state_len, the circular mode with cache_seqlens), "state indices for continuous
// batching" (the slot of a row), and the closing distinction between choosing another
// request's history, blocking history across packed samples, and continuing one request's
// history).  A row b uses slot s = indices[b] (b without indices):
//   conv history (oldest first): circular (p = cache_seqlens[b]) slots (p - j) mod state_len
//     for j = K-1 .. 1; linear: the row's last K-1 entries;
//   SSM initial state: ssm_pool[s];
// and after the prefill of its L tokens:
//   circular: new token i goes to slot (p + i) mod state_len (only the last state_len of them
//     can survive, so only those are written); linear: the row becomes the last state_len
//     entries of (old row ++ new tokens);
//   ssm_pool[s] = the final state.
// cache_seqlens is read, never advanced.  Rows whose slot lies outside [0, n_slots) run from
// zero states and store nothing.
#include "internal.h"

namespace ssm {
namespace {

template <class D>
__global__ void pool_gather_conv_kernel(const typename D::T* pool, const int32_t* indices,
                                        const int32_t* seqlens, typename D::T* hist,
                                        int64_t B, int64_t C, int64_t K, int64_t state_len,
                                        int64_t n_slots) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= B * C) return;
    const int64_t b = i / C, c = i % C;
    const int64_t s = indices ? static_cast<int64_t>(indices[b]) : b;
    const bool ok = s >= 0 && s < n_slots;
    for (int64_t j = 0; j < K - 1; ++j) {  // history position j, oldest first
        float v = 0.0f;
        if (ok) {
            int64_t slot;
            if (seqlens) {
                const int64_t back = (K - 1) - j;  // steps back from the write pointer
                slot = floor_mod(static_cast<int64_t>(seqlens[b]) - back, state_len);
            } else {
                slot = state_len - (K - 1) + j;
            }
            v = D::load(pool, (s * C + c) * state_len + slot);
        }
        D::store(hist, (b * C + c) * (K - 1) + j, v);
    }
}

// SSM states: block (x, y) moves elements 1024 x .. 1024 x + 1023 of the states of rows
// b = y, y + gridDim.y, ..., four per thread, as non-temporal 16-byte accesses when `vec`
// (per % 4 == 0 and both bases 16-byte aligned); a row's slot is looked up once per block
__global__ void __launch_bounds__(256) pool_gather_ssm_kernel(const float* pool,
                                                              const int32_t* indices, float* init,
                                                              int64_t B, int64_t per,
                                                              int64_t n_slots, bool vec) {
    const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (e >= per) return;
    for (int64_t b = blockIdx.y; b < B; b += gridDim.y) {
    const int64_t s = indices ? static_cast<int64_t>(indices[b]) : b;
    const bool ok = s >= 0 && s < n_slots;
    if (vec) {
        const f32x4_t v = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pool + s * per + e))
                             : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(init + b * per + e));
    } else {
        for (int64_t k = e; k < e + 4 && k < per; ++k) init[b * per + k] = ok ? pool[s * per + k] : 0.0f;
    }
    }
}

template <class D>
__global__ void pool_scatter_conv_kernel(typename D::T* pool, const int32_t* indices,
                                         const int32_t* seqlens, const typename D::T* x,
                                         int64_t B, int64_t L, int64_t C, int64_t state_len,
                                         int64_t n_slots) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= B * C) return;
    const int64_t b = i / C, c = i % C;
    const int64_t s = indices ? static_cast<int64_t>(indices[b]) : b;
    if (s < 0 || s >= n_slots) return;
    typename D::T* row = pool + (s * C + c) * state_len;
    if (seqlens) {
        const int64_t p = seqlens[b];
        const int64_t first = L > state_len ? L - state_len : 0;
        for (int64_t t = first; t < L; ++t)
            row[floor_mod(p + t, state_len)] = x[(b * L + t) * C + c];
    } else {
        // the last state_len entries of (old row ++ new tokens), in place: entry j comes from
        // old j + L (read ahead of every write) or from new token j + L - state_len
        for (int64_t j = 0; j < state_len; ++j)
            row[j] = j + L < state_len ? row[j + L] : x[(b * L + (j + L - state_len)) * C + c];
    }
}

__global__ void __launch_bounds__(256) pool_scatter_ssm_kernel(float* pool, const int32_t* indices,
                                                               const float* fin, int64_t B,
                                                               int64_t per, int64_t n_slots,
                                                               bool vec) {
    const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (e >= per) return;
    for (int64_t b = blockIdx.y; b < B; b += gridDim.y) {
    const int64_t s = indices ? static_cast<int64_t>(indices[b]) : b;
    if (s < 0 || s >= n_slots) continue;
    if (vec) {
        __builtin_nontemporal_store(
            __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(fin + b * per + e)),
            reinterpret_cast<f32x4_t*>(pool + s * per + e));
    } else {
        for (int64_t k = e; k < e + 4 && k < per; ++k) pool[s * per + k] = fin[b * per + k];
    }
    }
}

dim3 ssm_grid(int64_t batch, int64_t per) {
    return dim3(static_cast<unsigned>((per + 1023) / 1024),
                static_cast<unsigned>(batch < 65535 ? batch : 65535));
}
bool ssm_vec(const float* p, const float* q, int64_t per) {
    return per % 4 == 0 && ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(q)) & 15) == 0;
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

}  // namespace

hipError_t launch_pool_gather(const void* conv_pool, const float* ssm_pool, const int32_t* indices,
                              const int32_t* seqlens, void* conv_hist, float* ssm_init,
                              int64_t batch, int64_t C, int64_t K, int64_t state_len,
                              int64_t ssm_per, int64_t n_slots, ssm_dtype_t dtype,
                              hipStream_t stream) {
    if (dtype == SSM_BF16)
        pool_gather_conv_kernel<BF16><<<blocks_for(batch * C), 256, 0, stream>>>(
            static_cast<const uint16_t*>(conv_pool), indices, seqlens,
            static_cast<uint16_t*>(conv_hist), batch, C, K, state_len, n_slots);
    else
        pool_gather_conv_kernel<F32><<<blocks_for(batch * C), 256, 0, stream>>>(
            static_cast<const float*>(conv_pool), indices, seqlens, static_cast<float*>(conv_hist),
            batch, C, K, state_len, n_slots);
    if (batch > 0 && ssm_per > 0)
        pool_gather_ssm_kernel<<<ssm_grid(batch, ssm_per), 256, 0, stream>>>(
            ssm_pool, indices, ssm_init, batch, ssm_per, n_slots, ssm_vec(ssm_pool, ssm_init, ssm_per));
    return hipGetLastError();
}

hipError_t launch_pool_scatter(void* conv_pool, float* ssm_pool, const int32_t* indices,
                               const int32_t* seqlens, const void* x, const float* ssm_final,
                               int64_t batch, int64_t L, int64_t C, int64_t state_len,
                               int64_t ssm_per, int64_t n_slots, ssm_dtype_t dtype,
                               hipStream_t stream) {
    if (dtype == SSM_BF16)
        pool_scatter_conv_kernel<BF16><<<blocks_for(batch * C), 256, 0, stream>>>(
            static_cast<uint16_t*>(conv_pool), indices, seqlens, static_cast<const uint16_t*>(x),
            batch, L, C, state_len, n_slots);
    else
        pool_scatter_conv_kernel<F32><<<blocks_for(batch * C), 256, 0, stream>>>(
            static_cast<float*>(conv_pool), indices, seqlens, static_cast<const float*>(x), batch,
            L, C, state_len, n_slots);
    if (batch > 0 && ssm_per > 0)
        pool_scatter_ssm_kernel<<<ssm_grid(batch, ssm_per), 256, 0, stream>>>(
            ssm_pool, indices, ssm_final, batch, ssm_per, n_slots, ssm_vec(ssm_pool, ssm_final, ssm_per));
    return hipGetLastError();
}

}  // namespace ssm
