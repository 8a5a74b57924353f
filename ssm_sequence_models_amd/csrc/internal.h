// internal.h -- shared device helpers and launcher declarations of the HIP library.
// Not part of the public ABI (see include/ssm_mi355x.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_mi355x.h"

namespace ssm {

// ---------------------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// 8-byte accesses of data streamed once (read once or written once): non-temporal, so they do
// not displace what other blocks re-read; measured faster on plain 1 GiB copies
__device__ __forceinline__ uint2 ld_stream_u2(const uint16_t* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return uint2{v[0], v[1]};
}
__device__ __forceinline__ void st_stream_u2(uint16_t* p, uint2 v) {
    __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t*>(p));
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream_f4(const float4* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
// two floats -> two bf16 (nearest even) in one word, lo in bits 0-15 (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

struct F32 {
    using T = float;
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static float load(const T* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(T* p, int64_t i, float v) { p[i] = v; }
};
struct BF16 {
    using T = uint16_t;
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static float load(const T* p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(T* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// phi: identity or SiLU(z) = z / (1 + exp(-z)) with the hardware exp and reciprocal (about 2
// ulp); exp(-z) = inf gives -0 for very negative z
__device__ __forceinline__ float apply_act(float z, int act) {
    if (act == SSM_ACT_SILU) return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
    return z;
}

// Round a double to bf16, nearest even, without the double rounding of a plain
// double -> float -> bf16 chain: when the float lands exactly on a bf16 midpoint, the part
// the float dropped decides the direction.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
    const float f = static_cast<float>(v);
    const uint32_t b = __float_as_uint(f);
    if ((b & 0xFFFFu) == 0x8000u && static_cast<double>(f) != v) {
        const bool away = fabs(v) > fabs(static_cast<double>(f));
        return static_cast<uint16_t>((away ? b + 0x8000u : b - 0x8000u) >> 16);
    }
    return f32_to_bf16(f);
}

// bf16(phi(z)) for a conv sum z held in double (exact products of fp32 weights and 16-bit
// inputs), rounded as the exact phi(z) rounds.  SiLU runs in fp32.  To first order its
// relative error is below (7 + 3|z|) u, u = 2^-24: the rounding of z to fp32 through the
// condition number 1 + |z|; the rounding of the exp argument, which scales e^-z by up to
// 2|z| u; v_exp and v_rcp at one ulp (2u) each; and the roundings of 1 + e and of the
// product.  A relative error r is at most r / u ulps of the result, so results within
// 8 + 4|z| ulps of a bf16 rounding midpoint are recomputed in double and the rounding
// decision matches the exact value's.
__device__ __forceinline__ float silu_f32(double z, bool& near_midpoint) {
    const float zf = static_cast<float>(z);
    const float s = zf * __builtin_amdgcn_rcpf(1.0f + __expf(-zf));
    // distance, in fp32 ulps, of s from the bf16 rounding midpoint: |low 16 bits - 0x8000|
    // (exact in float; compiles to one add, one convert and the compare)
    const float lo = static_cast<float>(__float_as_uint(s) & 0xFFFFu);
    near_midpoint = fabsf(lo - 32768.0f) <= 8.0f + 4.0f * fabsf(zf);
    return s;
}
__device__ __forceinline__ uint16_t silu_f64_to_bf16(double z) {
    return f64_to_bf16(z / (1.0 + exp(-z)));
}
__device__ __forceinline__ uint16_t act_to_bf16(double z, int act) {
    if (act != SSM_ACT_SILU) return f64_to_bf16(z);
    bool near;
    const float s = silu_f32(z, near);
    return near ? silu_f64_to_bf16(z) : f32_to_bf16(s);
}
// The same for NB values at once: all fast paths first (independent chains the scheduler
// can interleave), then a single branch for the rare near-midpoint recomputations.
template <int NB>
__device__ __forceinline__ void act_to_bf16_batch(const double (&z)[NB], int act,
                                                  uint16_t (&out)[NB]) {
    if (act != SSM_ACT_SILU) {
#pragma unroll
        for (int e = 0; e < NB; ++e) out[e] = f64_to_bf16(z[e]);
        return;
    }
    uint32_t near_mask = 0;
#pragma unroll
    for (int e = 0; e < NB; ++e) {
        bool near;
        const float s = silu_f32(z[e], near);
        out[e] = f32_to_bf16(s);
        near_mask |= static_cast<uint32_t>(near) << e;
    }
    if (near_mask != 0) {
#pragma unroll
        for (int e = 0; e < NB; ++e)
            if (near_mask & (1u << e)) out[e] = silu_f64_to_bf16(z[e]);
    }
}

__host__ __device__ __forceinline__ int64_t floor_mod(int64_t a, int64_t m) {
    int64_t r = a % m;
    return r < 0 ? r + m : r;
}

// ---------------------------------------------------------------------------------------
// launchers (return hipSuccess or the launch error); arguments are validated by the ABI
// ---------------------------------------------------------------------------------------
hipError_t launch_conv1d_fwd(const void* x, const float* w, const float* bias,
                             const void* init_state, void* final_state, const int32_t* seq_idx,
                             void* out, int64_t B, int64_t L, int64_t C, int64_t K,
                             ssm_dtype_t dtype, int act, hipStream_t stream);

hipError_t launch_conv1d_update(const void* x, void* pool, const float* w, const float* bias,
                                const int32_t* indices, const int32_t* cache_seqlens, void* out,
                                int64_t B, int64_t C, int64_t L_new, int64_t K,
                                int64_t state_len, int64_t n_slots, ssm_dtype_t dtype, int act,
                                hipStream_t stream);

// Recurrent (token-sequential) scan used by ssm_step and as the general-shape scan path.
struct RecurrentArgs {
    const void* x;
    int64_t x_sb, x_st, x_sc;
    const float* dt;  // [B, T, H]
    const float* A;   // [H]
    const void* Bm;
    int64_t B_sb, B_st, B_sc;
    const void* Cm;
    int64_t C_sb, C_st, C_sc;
    const float* state_in;    // base of [slots or B, H, P, N] (NULL -> zeros)
    float* state_out;         // base of [slots or B, H, P, N] (NULL -> not written)
    const int32_t* indices;   // [B] slot per row or NULL (slot = b)
    int64_t n_slots;          // bound for indices (rows outside are skipped, y zeroed)
    const int32_t* seq_idx;   // [B, T] or NULL
    void* y;                  // [B, T, H, P]
    int64_t B, T, H, P, G, N;
    // diagonal (per-state-dimension) transition: log a_t[n] from log_decay [B, T, H, N], or
    // dt_t A_vec[h][n] from A_vec [H, N]; both NULL = the scalar exp(dt_t A[h])
    const float* log_decay;
    const float* A_vec;
};
bool recurrent_supported(int64_t P, int64_t N, bool vector_decay = false);
hipError_t launch_recurrent(const RecurrentArgs& a, ssm_dtype_t dtype, hipStream_t stream);
// the diagonal-transition scan for long rows (headdim 64, dstate 64 or 128; contiguous
// states, 16-byte aligned); launch_recurrent covers the other shapes
bool vdecay_supported(int64_t P, int64_t N);
hipError_t launch_vdecay(const RecurrentArgs& a, ssm_dtype_t dtype, hipStream_t stream);
// the chunked (matrix-core) form of the diagonal-transition scan: gate form, bf16, headdim 64,
// dstate 128, contiguous 16-byte aligned rows, no slot map (launch_vdecay dispatches to it)
bool vchunk_supported(const RecurrentArgs& a, ssm_dtype_t dtype);
hipError_t launch_vchunk(const RecurrentArgs& a, hipStream_t stream);

// Chunked (SSD) scan on MFMA for bf16 inputs with headdim 64, dstate 128.
bool chunked_supported(int64_t P, int64_t N, ssm_dtype_t dtype);
size_t chunked_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t G, int64_t N);
struct ChunkedArgs {
    // x channels: element (b, t, h*P + p) at x[(b*L + t)*x_row + x_col0 + h*P + p]  (bf16)
    const uint16_t* x;
    int64_t x_row, x_col0;
    // B / C channels: element (b, t, g, n) at src[(b*L + t)*row + col0 + g*N + n]  (bf16);
    // in the fused call both point into xBC, otherwise at the Bm / Cm arrays
    const uint16_t* bsrc;
    int64_t b_row, b_col0;
    const uint16_t* csrc;
    int64_t c_row, c_col0;
    // fused conv (x_col0 = 0, b_col0 = H*P, c_col0 = H*P + G*N inside xBC rows of C_conv)
    bool fused_conv;
    const float* conv_w;        // [C_conv, K]
    const float* conv_b;        // [C_conv] or NULL
    const uint16_t* conv_init;  // [B, C_conv, K-1] or NULL
    uint16_t* conv_final;       // [B, C_conv, K-1] or NULL
    int64_t C_conv, K;
    int act;
    const float* dt;            // [B, L, H]
    const float* A;             // [H]
    const float* init_state;    // [B, H, P, N] or NULL (rows: see state_slots)
    float* final_state;         // [B, H, P, N] or NULL
    // With n_state_slots > 0 the states are rows of [n_state_slots, H, P, N]: row b's at
    // s = state_slots[b] (s = b without state_slots); a row whose s lies outside
    // [0, n_state_slots) starts from zero and stores no final state
    const int32_t* state_slots;
    int64_t n_state_slots;
    const int32_t* seq_idx;     // [B, L] or NULL
    uint16_t* y;                // [B, L, H, P]
    int64_t B, L, H, P, G, N;
    void* workspace;            // chunked_workspace_bytes(B, L, H, G, N)
    // Set by launch_chunked.  Rows with few heads split into nseg segments of seg_chunks
    // chunks run side by side: seg_state [B, H, nseg, P, N] holds in slot 0 the initial state
    // and in slot s >= 1 segment s-1's local end state from a zero start; seg_decay [B, H, nseg]
    // each segment's decay product.
    int64_t nseg, seg_chunks;
    float* seg_state;
    float* seg_decay;
};
hipError_t launch_chunked(const ChunkedArgs& a, hipStream_t stream, hipEvent_t ev_before_main,
                          hipEvent_t ev_after_main);

// small helpers
int64_t conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t channels, int64_t width);
hipError_t launch_conv1d_bwd(const void* x, const float* w, const float* bias, const void* init,
                             const int32_t* seq, const void* dy, const void* dfin, void* dx,
                             void* dinit, float* dw, float* dbias, void* workspace,
                             int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                             ssm_dtype_t dtype, ssm_act_t act, hipStream_t stream);
hipError_t launch_scan_bwd_h0(const float* dt, const float* A, const void* Cm,
                              const int32_t* seq, const void* dy, const float* dfin, float* dh0,
                              int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t ngroups, int64_t dstate, ssm_dtype_t dtype,
                              hipStream_t stream);
hipError_t launch_pool_gather(const void* conv_pool, const float* ssm_pool, const int32_t* indices,
                              const int32_t* seqlens, void* conv_hist, float* ssm_init,
                              int64_t batch, int64_t C, int64_t K, int64_t state_len,
                              int64_t ssm_per, int64_t n_slots, ssm_dtype_t dtype,
                              hipStream_t stream);
hipError_t launch_pool_scatter(void* conv_pool, float* ssm_pool, const int32_t* indices,
                               const int32_t* seqlens, const void* x, const float* ssm_final,
                               int64_t batch, int64_t L, int64_t C, int64_t state_len,
                               int64_t ssm_per, int64_t n_slots, ssm_dtype_t dtype,
                               hipStream_t stream);
hipError_t launch_state_stats(const float* fin, int64_t B, int64_t H, int64_t per, double beta,
                              float* mean, float* var, hipStream_t stream);
hipError_t launch_state_noise(float* out, int64_t n, int64_t H, int64_t per, const float* mean,
                              const float* var, float sigma, uint64_t seed, uint64_t offset,
                              hipStream_t stream);
int64_t state_reset_blocks(int64_t B, int64_t row_bytes, int unit);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_state_reset(const void* src, void* dst, uint8_t* mask, int64_t B,
                              int64_t row_bytes, int unit, uint64_t threshold, uint64_t seed,
                              uint64_t offset, hipStream_t stream);
hipError_t launch_copy_or_zero_f32(float* dst, const float* src, int64_t n, hipStream_t s);
hipError_t launch_copy_or_zero_bytes(void* dst, const void* src, int64_t nbytes, hipStream_t s);

}  // namespace ssm
