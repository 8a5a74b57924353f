// init_state.hip -- initial-state distributions for training with non-zero initial states
// (length-generalization reading notes, Sec. 2.6: the table of four interventions, the
// Fitted Noise update Eqs. (5)-(6), and State Passing with its occasional reset):
//   state_stats_kernel   per head, Mean and (population) Variance of the final states over
//                        batch rows, channels and state dimension, blended into running
//                        statistics with the new batch weighted 1 - beta;
//   noise_kernel         Fitted Noise (N(mean[h], var[h]) per head) or Random Noise
//                        (N(0, sigma^2)) initial states;
//   reset_kernel         State Passing's reset: each row zeroed with probability p.
// Random numbers: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011) with key (seed, purpose) and counter (block, offset, 0, 0);
// purpose 0 is the Gaussian noise (Box-Muller on 24 bits of each half of a word: eight
// normals per block), purpose 1 the reset decisions (top 32 bits of one word against
// floor(p 2^32)).
#include <algorithm>

#include "internal.h"

namespace ssm {
namespace {

struct U64x4 {
    uint64_t v[4];
};

// The full 128-bit product m c from four 32 x 32 -> 64-bit partial products, shared by both
// halves (a separate high product and 64-bit low product recompute some of them).  No sum
// overflows: (2^32 - 1)^2 + 2 (2^32 - 1) < 2^64.
__device__ __forceinline__ void mul128(uint64_t m, uint64_t c, uint64_t& hi, uint64_t& lo) {
    const uint64_t ml = static_cast<uint32_t>(m), mh = m >> 32;
    const uint64_t cl = static_cast<uint32_t>(c), ch = c >> 32;
    const uint64_t ll = ml * cl;
    const uint64_t t = ml * ch + (ll >> 32);
    const uint64_t u = mh * cl + static_cast<uint32_t>(t);
    hi = mh * ch + (t >> 32) + (u >> 32);
    lo = (u << 32) | static_cast<uint32_t>(ll);
}

// ten rounds: multiply counter words 0 and 2 by the two round constants, swap the 128-bit
// products' halves into the new counter with the round key mixed into the high halves, and
// advance the key by the Weyl increments between rounds
__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                               uint64_t c3, uint64_t k0, uint64_t k1) {
    constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
    constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t hi0, lo0, hi1, lo1;
        mul128(kM0, c0, hi0, lo0);
        mul128(kM1, c2, hi1, lo1);
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kW0;
        k1 += kW1;
    }
    return U64x4{{c0, c1, c2, c3}};
}

// Box-Muller on one 64-bit word: u1 = (bits 40-63 + 1) 2^-24 in (0, 1], u2 = (bits 8-31)
// 2^-24 in [0, 1) (24 bits of each 32-bit half, both exact in fp32); r = sqrt(-2 ln u1);
// (r cos 2 pi u2, r sin 2 pi u2).  sincospi takes 2 u2 (exact), so the angle is not rounded
// through 2 pi.
__device__ __forceinline__ void box_muller(uint64_t w, float& z0, float& z1) {
    const float u1 = static_cast<float>(static_cast<uint32_t>(w >> 40) + 1u) * 0x1p-24f;
    const float u2 = static_cast<float>(static_cast<uint32_t>(w >> 8) & 0xFFFFFFu) * 0x1p-24f;
    const float r = sqrtf(-2.0f * logf(u1));
    float s, c;
    sincospif(2.0f * u2, &s, &c);
    z0 = r * c;
    z1 = r * s;
}

constexpr int kStatsThreads = 1024;

// fixed-order block sum of one double per thread (deterministic)
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < kStatsThreads / 64; ++w) t += red[w];
    __syncthreads();
    return t;  // meaningful in thread 0
}

// one block per head, one pass: sums of d = x - s and d^2 in double, s = the head's first
// value (shifting by a value of the data keeps the variance exact to double rounding however
// large the common offset), then mean = s + S1 / n and Var = (S2 - S1^2 / n) / n.  Four
// 16-byte loads per thread are in flight per row.
__global__ __launch_bounds__(kStatsThreads) void state_stats_kernel(
    const float* fin, int64_t B, int64_t H, int64_t per, double beta, float* mean, float* var) {
    __shared__ double red[kStatsThreads / 64];
    const int64_t h = blockIdx.x;
    const bool vec = (per % 4) == 0 && (reinterpret_cast<uintptr_t>(fin) & 15) == 0;
    const double shift = fin[h * per];
    double s1 = 0.0, s2 = 0.0;
    auto acc4 = [&](const float4 q) {
        const double d0 = q.x - shift, d1 = q.y - shift, d2 = q.z - shift, d3 = q.w - shift;
        s1 += (d0 + d1) + (d2 + d3);
        s2 += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    };
    int64_t b0 = 0;
    if (vec) {
        // four rows at a time, so each thread has several 16-byte loads in flight (a head's
        // slice of one row is only a couple of loads per thread)
        const int64_t n4 = per / 4;
        for (; b0 + 4 <= B; b0 += 4) {
            for (int64_t i = threadIdx.x; i < n4; i += kStatsThreads) {
                float4 q[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    q[r] = ld_stream_f4(reinterpret_cast<const float4*>(fin + ((b0 + r) * H + h) * per) + i);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc4(q[r]);
            }
        }
    }
    for (int64_t b = b0; b < B; ++b) {
        const float* row = fin + (b * H + h) * per;
        if (vec) {
            const float4* r4 = reinterpret_cast<const float4*>(row);
            const int64_t n4 = per / 4;
#pragma unroll 4
            for (int64_t i = threadIdx.x; i < n4; i += kStatsThreads) acc4(ld_stream_f4(r4 + i));
        } else {
            for (int64_t i = threadIdx.x; i < per; i += kStatsThreads) {
                const double d = row[i] - shift;
                s1 += d;
                s2 += d * d;
            }
        }
    }
    s1 = block_sum(s1, red);
    s2 = block_sum(s2, red);
    if (threadIdx.x == 0) {
        const double n = static_cast<double>(B * per);
        const double m = shift + s1 / n;
        double v = (s2 - s1 * (s1 / n)) / n;
        v = v > 0.0 ? v : 0.0;
        mean[h] = static_cast<float>((1.0 - beta) * m + beta * static_cast<double>(mean[h]));
        var[h] = static_cast<float>((1.0 - beta) * v + beta * static_cast<double>(var[h]));
    }
}

// one thread per Philox block = eight consecutive elements (pair j from word j)
__global__ __launch_bounds__(256) void noise_kernel(float* out, int64_t n, int64_t H, int64_t per,
                                                    const float* mean, const float* var,
                                                    float sigma, uint64_t seed, uint64_t offset) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t e0 = 8 * i;
    if (e0 >= n) return;
    const U64x4 w = philox4x64_10(static_cast<uint64_t>(i), offset, 0, 0, seed, 0);
    float z[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) box_muller(w.v[j], z[2 * j], z[2 * j + 1]);
    if (mean) {
        // one 64-bit division per thread: with per >= 8 the eight elements span at most two
        // heads, h0 and the next one
        const int64_t q = e0 / per, rem = e0 - q * per, h0 = q % H;
        const int64_t h1 = h0 + 1 == H ? 0 : h0 + 1;
        const float m0 = mean[h0], s0 = sqrtf(var[h0]);
        const float m1 = mean[h1], s1 = sqrtf(var[h1]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (per >= 8) {
                const bool next = rem + j >= per;
                z[j] = (next ? m1 : m0) + (next ? s1 : s0) * z[j];
            } else {
                const int64_t h = ((e0 + j) / per) % H;
                z[j] = mean[h] + sqrtf(var[h]) * z[j];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = sigma * z[j];
    }
    if (e0 + 7 < n && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        f32x4_t* o = reinterpret_cast<f32x4_t*>(out + e0);
        __builtin_nontemporal_store(f32x4_t{z[0], z[1], z[2], z[3]}, o);
        __builtin_nontemporal_store(f32x4_t{z[4], z[5], z[6], z[7]}, o + 1);
    } else {
        for (int j = 0; j < 8 && e0 + j < n; ++j) out[e0 + j] = z[j];
    }
}

// row = blockIdx.x / blocks_per_row; every thread derives the row's decision itself (one
// Philox block), then copies or zeroes its units of the row
template <class U>
__global__ __launch_bounds__(256) void reset_kernel(const U* src, U* dst, uint8_t* mask,
                                                    int64_t units, int64_t blocks_per_row,
                                                    uint64_t threshold, uint64_t seed,
                                                    uint64_t offset) {
    const int64_t b = blockIdx.x / blocks_per_row;
    const int64_t chunk = blockIdx.x % blocks_per_row;
    const U64x4 w = philox4x64_10(static_cast<uint64_t>(b / 4), offset, 0, 0, seed, 1);
    const bool zero = (w.v[b % 4] >> 32) < threshold;
    if (mask && chunk == 0 && threadIdx.x == 0) mask[b] = zero ? 1 : 0;
    if (!zero && src == dst) return;  // in place: kept rows stay as they are
    const int64_t base = b * units;
    constexpr int kItems = 4;
    const int64_t start = chunk * (256 * kItems) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int64_t u = start + k * 256;
        if (u < units) __builtin_nontemporal_store(zero ? U{} : __builtin_nontemporal_load(src + base + u), dst + base + u);
    }
}

// A plain device-to-device copy with non-temporal 16-byte accesses, four units per thread in
// flight: the streaming reference the benchmark sets beside the HBM peak.  Bytes past the last
// whole unit (and every byte of a copy whose pointers are not 16-byte aligned) go one at a time.
__global__ void __launch_bounds__(256) stream_copy_kernel(const u32x4_t* src, u32x4_t* dst,
                                                          int64_t units) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 1024;
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x; i0 < units; i0 += stride) {
        u32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + 256 * u < units) v[u] = __builtin_nontemporal_load(src + i0 + 256 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + 256 * u < units) __builtin_nontemporal_store(v[u], dst + i0 + 256 * u);
    }
}

__global__ void __launch_bounds__(256) byte_copy_kernel(const uint8_t* src, uint8_t* dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
    const int64_t units = (a & 15) == 0 ? bytes / 16 : 0;
    if (units > 0) {
        const int64_t blocks = std::min<int64_t>((units + 1023) / 1024, 16384);
        stream_copy_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
            static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), units);
    }
    const int64_t rest = bytes - 16 * units;
    if (rest > 0) {
        const int64_t blocks = std::min<int64_t>((rest + 255) / 256, 16384);
        byte_copy_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
            static_cast<const uint8_t*>(src) + 16 * units, static_cast<uint8_t*>(dst) + 16 * units, rest);
    }
    return hipGetLastError();
}

hipError_t launch_state_stats(const float* fin, int64_t B, int64_t H, int64_t per, double beta,
                              float* mean, float* var, hipStream_t stream) {
    state_stats_kernel<<<static_cast<unsigned>(H), kStatsThreads, 0, stream>>>(fin, B, H, per, beta,
                                                                              mean, var);
    return hipGetLastError();
}

hipError_t launch_state_noise(float* out, int64_t n, int64_t H, int64_t per, const float* mean,
                              const float* var, float sigma, uint64_t seed, uint64_t offset,
                              hipStream_t stream) {
    const int64_t threads = (n + 7) / 8;
    noise_kernel<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, stream>>>(
        out, n, H, per, mean, var, sigma, seed, offset);
    return hipGetLastError();
}

int64_t state_reset_blocks(int64_t B, int64_t row_bytes, int unit) {
    const int64_t units = row_bytes / unit;
    const int64_t bpr = units > 0 ? (units + 1023) / 1024 : 1;
    return B * bpr;
}

hipError_t launch_state_reset(const void* src, void* dst, uint8_t* mask, int64_t B,
                              int64_t row_bytes, int unit, uint64_t threshold, uint64_t seed,
                              uint64_t offset, hipStream_t stream) {
    const int64_t units = row_bytes / unit;
    const int64_t bpr = units > 0 ? (units + 1023) / 1024 : 1;
    const unsigned grid = static_cast<unsigned>(B * bpr);
    if (unit == 16)
        reset_kernel<u32x4_t><<<grid, 256, 0, stream>>>(static_cast<const u32x4_t*>(src),
                                                         static_cast<u32x4_t*>(dst), mask, units, bpr,
                                                         threshold, seed, offset);
    else if (unit == 4)
        reset_kernel<uint32_t><<<grid, 256, 0, stream>>>(static_cast<const uint32_t*>(src),
                                                         static_cast<uint32_t*>(dst), mask, units,
                                                         bpr, threshold, seed, offset);
    else
        reset_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(src),
                                                         static_cast<uint16_t*>(dst), mask, units,
                                                         bpr, threshold, seed, offset);
    return hipGetLastError();
}

}  // namespace ssm
