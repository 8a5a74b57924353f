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
//  * ssd_prep_kernel, one block per (batch row, chunk, group): the conv (+phi, rounded to
//    bf16 as the exact value rounds) over the chunk's B and C channels, once for all heads of
//    the group; writes C (token-major), B (channel-major) and G = C B^T (fp32, MFMA) to the
//    workspace.  Doing this per head would repeat the B/C conv nheads times.
//  * ssd_main_kernel, one block per (batch row, head) with 12 wavefronts, three per SIMD:
//      - 4 consumer waves each own 16 of the 64 head channels and keep their [16 x 128] slice
//        of the fp32 state in MFMA accumulators for the whole sequence.  Per chunk they issue
//        the contractions on v_mfma_f32_16x16x32_bf16:
//            Y^T += h-slice x C^T      (initial-state part)
//            Y^T += X^T x M^T          (intra-chunk part, M = G o decay mask)
//            h^T += B^T x (W o X)      (state update)
//        The fp32 operands (h, M, W o X) enter as a hi + lo pair of bf16 (v = hi + lo with
//        |v - hi - lo| <= 2^-17 |v|); the other operand (x, B, C) is exact in bf16, so each
//        contraction is accurate to about fp32 at the bf16 MFMA rate.
//      - 4 producer waves run one chunk ahead: move the next chunk's C / B^T tiles and the
//        raw x rows of the chunk after it from L2 / HBM straight into LDS, compute the
//        in-chunk cumulative log-decay (a DPP prefix scan per wavefront) and the M tiles,
//        and store the previous chunk's y rows.
//      - 4 conv waves run the register-window conv + SiLU of the head's x channels for the
//        next chunk from the staged raw rows; each lane's 16 outputs are exactly the X
//        operand of the consumer lane with the same index.
//    One block barrier per chunk hands the double-buffered LDS stages over.
#include "internal.h"

namespace ssm {
namespace {

constexpr int kQ = 64;       // tokens per chunk
constexpr int kP = 64;       // head channels (4 consumer waves x 16)
constexpr int kN = 128;      // state size
constexpr int kKmax = 8;     // widest conv handled
constexpr int kPrepThreads = 1024;
constexpr int kMainThreads = 768;  // 4 consumer, 4 producer and 4 conv wavefronts

// workspace per (row, chunk, group)
constexpr int64_t kWsC = static_cast<int64_t>(kQ) * kN;    // bf16 elements, [token][n]
constexpr int64_t kWsBt = static_cast<int64_t>(kN) * kQ;   // bf16 elements, [n][token]
constexpr int64_t kWsG = static_cast<int64_t>(kQ) * kQ;    // fp32 elements, [i][j]

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t* base, int off) {
    return *reinterpret_cast<const T*>(base + off);
}
template <class T>
__device__ __forceinline__ void lds_st(uint8_t* base, int off, const T& v) {
    *reinterpret_cast<T*>(base + off) = v;
}

// v = hi + lo, hi = rne(v), lo = rne(v - hi): one paired conversion for two his, then
// lo = v - hi in one instruction per value: the bf16 dot product of the hi pair with (-1, 0)
// or (0, -1), accumulated onto v (the difference is exact in fp32, so the dot product's
// rounding does not enter; checked bit for bit against the subtraction on the GPU).  The two
// constant pairs go in as register values the compiler cannot see: as a source of this
// instruction it encodes 0x0000BF80 as the inline constant -1.0, which the hardware reads as
// the 32-bit pattern of -1.0f, the pair (0, -1).
__device__ __forceinline__ void split_hilo(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    uint32_t c_lo = 0x0000BF80u, c_hi = 0xBF800000u;
    asm volatile("" : "+s"(c_lo), "+s"(c_hi));
    const bf16x2v neg_lo = __builtin_bit_cast(bf16x2v, c_lo);  // (-1, 0)
    const bf16x2v neg_hi = __builtin_bit_cast(bf16x2v, c_hi);  // (0, -1)
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t hp = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        const bf16x2v hv = __builtin_bit_cast(bf16x2v, hp);
        h[e] = hp;
        l[e] = pack_bf16x2(__builtin_amdgcn_fdot2_f32_bf16(hv, neg_lo, v[2 * e], false),
                           __builtin_amdgcn_fdot2_f32_bf16(hv, neg_hi, v[2 * e + 1], false));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ void split_hilo4(const float (&v)[4], u32x2& hi, u32x2& lo) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    uint32_t c_lo = 0x0000BF80u, c_hi = 0xBF800000u;
    asm volatile("" : "+s"(c_lo), "+s"(c_hi));
    const bf16x2v neg_lo = __builtin_bit_cast(bf16x2v, c_lo);  // (-1, 0)
    const bf16x2v neg_hi = __builtin_bit_cast(bf16x2v, c_hi);  // (0, -1)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const uint32_t hp = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        const bf16x2v hv = __builtin_bit_cast(bf16x2v, hp);
        hi[e] = hp;
        lo[e] = pack_bf16x2(__builtin_amdgcn_fdot2_f32_bf16(hv, neg_lo, v[2 * e], false),
                            __builtin_amdgcn_fdot2_f32_bf16(hv, neg_hi, v[2 * e + 1], false));
    }
}

// Inclusive prefix over the 64 lanes of a wavefront with DPP: row_shr 1/2/4/8 inside each
// row of 16 lanes, then row_bcast 15 / 31 carry the row totals forward.
__device__ __forceinline__ float wave_incl_sum(float v) {
    const int z = __float_as_int(0.0f);
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x118, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(z, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}
__device__ __forceinline__ int wave_incl_max(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x111, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x112, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x114, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x118, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x142, 0xa, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(-1, v, 0x143, 0xc, 0xf, false));
    return v;
}

// The state-only pass of a segment (its end state from a zero start) may begin at the last
// chunk c from which the segment's remaining log-decay sum S(c) = sum of dt_t A over the
// tokens from chunk c to the segment end is below -208: every token before chunk c then
// reaches the end state with a factor exp(sum of its later dt A) <= exp(S(c)) < 1e-90, as
// long as each skipped token has dt A <= 0, which is checked (a NaN or positive dt A among
// them keeps the whole segment).  The skipped tokens' part of the end state is below fp32's
// smallest subnormal for any state of magnitude up to 1e44; the segment's decay product is
// then exactly 0 in fp32 as well.  Returns the number of chunks to skip (0: none).  All
// threads of the block call it; it uses 66 floats of LDS at scr and ends with a barrier.
template <int NT>
__device__ int64_t state_pass_skip(const float* dtc, int64_t H, int64_t L, int64_t c0,
                                   int64_t nCl, float A, float* scr, int tid) {
    constexpr int NW = NT / 64;
    constexpr int PER = (64 + NW - 1) / NW;  // chunks per wave in a window of 64
    constexpr float kCut = -208.0f;
    const int wave = tid >> 6, lane = tid & 63;
    int64_t hit = -1;  // chunk index (in the segment) of the last crossing
    float carry = 0.0f;
    for (int64_t w0 = nCl; w0 > 0; w0 -= 64) {
        // chunk sums of dt A for the window's chunks w0 - 1 - l (l < 64) into scr[l]
        const int nw = static_cast<int>(min<int64_t>(64, w0));
        float v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int l = wave + NW * i;
            const int64_t t = (c0 + w0 - 1 - l) * kQ + lane;
            v[i] = (l < nw && t < L) ? dtc[t * H] * A : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int l = wave + NW * i;
            const float sum = wave_incl_sum(v[i]);
            if (l < nw && lane == 63) scr[l] = sum;
        }
        __syncthreads();
        if (wave == 0) {
            // lane l: the sum from chunk w0 - 1 - l to the segment end
            const float S = wave_incl_sum(lane < nw ? scr[lane] : 0.0f) + carry;
            const uint64_t m = __ballot(lane < nw && S < kCut);
            const float tot = __shfl(S, 63);
            if (lane == 0) {
                scr[64] = m ? static_cast<float>(__builtin_ctzll(m)) : -1.0f;
                scr[65] = tot;
            }
        }
        __syncthreads();
        const float r = scr[64];
        carry = scr[65];
        __syncthreads();  // scr is rewritten by the next window
        if (r >= 0.0f) {
            hit = w0 - 1 - static_cast<int64_t>(r);
            break;
        }
    }
    if (hit <= 0) return 0;
    // every skipped token must have dt A <= 0 (not NaN, not positive)
    int bad = 0;
    const int64_t t_end = (c0 + hit) * kQ;
#pragma unroll 4
    for (int64_t t = c0 * kQ + tid; t < t_end; t += NT) bad |= !(dtc[t * H] * A <= 0.0f);
    return __syncthreads_or(bad) ? 0 : hit;
}

__device__ __forceinline__ int64_t ws_unit(const ChunkedArgs& a, int64_t b, int64_t c,
                                           int64_t g, int64_t nC) {
    return (b * nC + c) * a.G + g;
}

// =======================================================================================
// prep: conv + bf16 rounding of the B / C channels of one (row, chunk, group), then
// C token-major, B channel-major and G = C B^T into the workspace
// =======================================================================================
constexpr int kPrepStride = kN * 2 + 16;   // [token][n] bf16 rows in LDS (conv outputs)
constexpr int kPrepRaw = 2 * kN * 2 + 16;  // [row][B n | C n] bf16 raw input rows in LDS
constexpr int kPrepLds = 2 * kQ * kPrepStride + (kQ + kKmax - 1) * kPrepRaw + 72 * 4;

template <int K>
__global__ void __launch_bounds__(kPrepThreads)
ssd_prep_kernel(ChunkedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[kPrepLds];
    constexpr int kRows = kQ + K - 1;
    uint8_t* sB = sm;
    uint8_t* sC = sm + kQ * kPrepStride;
    uint8_t* sRaw = sm + 2 * kQ * kPrepStride;
    int32_t* sSeq = reinterpret_cast<int32_t*>(sRaw + (kQ + kKmax - 1) * kPrepRaw);

    const int tid = threadIdx.x;
    const int64_t cn = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int64_t L = a.L;
    const int64_t nC = (L + kQ - 1) / kQ;
    const int64_t t0 = cn * kQ;
    const bool has_seq = a.seq_idx != nullptr;

    if (has_seq && tid < kRows) {
        int64_t t = t0 - (K - 1) + tid;
        t = t < 0 ? 0 : (t >= L ? L - 1 : t);
        sSeq[tid] = a.seq_idx[b * L + t];
    }
    // raw rows t0-(K-1) .. t0+Q-1 of the group's B and C channels, 16 bytes per load
    // (B and C channels of a group are each 128 contiguous bf16 of a token row).  A thread's
    // pieces are all loaded before any is stored: each load reads a row clamped into
    // 0 .. L-1, so none sits behind a branch, and a select drops the clamped ones afterwards.
    constexpr int kPieces = kRows * 32;
    constexpr int kPer = (kPieces + kPrepThreads - 1) / kPrepThreads;
    u32x4 raw[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = min(tid + i * kPrepThreads, kPieces - 1);
        const int rho = idx >> 5, piece = idx & 31;
        const bool isC = piece >= 16;
        const int64_t t = t0 - (K - 1) + rho;
        const int64_t tc = t < 0 ? 0 : (t >= L ? L - 1 : t);
        const int64_t row = isC ? a.c_row : a.b_row;
        const int64_t col = (isC ? a.c_col0 : a.b_col0) + g * kN + (piece & 15) * 8;
        raw[i] = *reinterpret_cast<const u32x4*>((isC ? a.csrc : a.bsrc) + (b * L + tc) * row + col);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = tid + i * kPrepThreads;
        if (idx >= kPieces) break;
        const int rho = idx >> 5, piece = idx & 31;
        const int64_t t = t0 - (K - 1) + rho;
        u32x4 v = t >= 0 && t < L ? raw[i] : u32x4{0u, 0u, 0u, 0u};
        if (t < 0 && a.fused_conv && a.conv_init) {
            const bool isC = piece >= 16;
            const int64_t col = (isC ? a.c_col0 : a.b_col0) + g * kN + (piece & 15) * 8;
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = a.conv_init[(b * a.C_conv + col + 2 * e) * (K - 1) + (K - 1) + t];
                const uint32_t hi = a.conv_init[(b * a.C_conv + col + 2 * e + 1) * (K - 1) + (K - 1) + t];
                w4[e] = lo | (hi << 16);
            }
            v = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
        lds_st(sRaw, rho * kPrepRaw + piece * 16, v);
    }
    __syncthreads();

    // one channel and one quarter of the chunk per thread (B channels 0..127, then C channels;
    // tokens 16 qt .. 16 qt + 15), 8 tokens per batch
    static_assert(kPrepThreads == 8 * kN, "four threads per conv channel");
    {
        const int ch = tid & (2 * kN - 1), qt = tid / (2 * kN);
        const bool isC = ch >= kN;
        const int n = isC ? ch - kN : ch;
        const int64_t col = (isC ? a.c_col0 : a.b_col0) + g * kN + n;
        uint8_t* dst = isC ? sC : sB;
        if (a.fused_conv) {
            double w[K];
#pragma unroll
            for (int k = 0; k < K; ++k) w[k] = a.conv_w[col * K + k];
            const double bias = a.conv_b ? a.conv_b[col] : 0.0f;
            for (int j0 = qt * (kQ / 4); j0 < (qt + 1) * (kQ / 4); j0 += 8) {
                double u[8 + K - 1];
                int32_t id[8 + K - 1];
#pragma unroll
                for (int tau = 0; tau < 8 + K - 1; ++tau) {
                    u[tau] = bf16_to_f32(lds_ld<uint16_t>(sRaw, (j0 + tau) * kPrepRaw + ch * 2));
                    id[tau] = has_seq ? sSeq[j0 + tau] : 0;
                }
                double z[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    z[e] = bias;
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const double tap = (!has_seq || id[e + k] == id[e + K - 1]) ? u[e + k] : 0.0;
                        z[e] = fma(w[k], tap, z[e]);
                    }
                }
                uint16_t o[8];
                act_to_bf16_batch(z, a.act, o);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t v = t0 + j0 + e < L ? o[e] : uint16_t(0);
                    *reinterpret_cast<uint16_t*>(dst + (j0 + e) * kPrepStride + n * 2) = v;
                }
            }
        } else {
            for (int j = qt * (kQ / 4); j < (qt + 1) * (kQ / 4); ++j)
                *reinterpret_cast<uint16_t*>(dst + j * kPrepStride + n * 2) =
                    lds_ld<uint16_t>(sRaw, (j + K - 1) * kPrepRaw + ch * 2);
        }
    }
    __syncthreads();

    const int64_t unit = ws_unit(a, b, cn, g, nC);
    uint16_t* wsC = static_cast<uint16_t*>(a.workspace);
    uint16_t* wsBt = wsC + a.B * nC * a.G * kWsC;
    float* wsG = reinterpret_cast<float*>(wsBt + a.B * nC * a.G * kWsBt);
    for (int idx = tid; idx < kQ * kN / 8; idx += kPrepThreads) {
        const int i = idx >> 4, q = idx & 15;
        *reinterpret_cast<u32x4*>(wsC + unit * kWsC + i * kN + q * 8) =
            lds_ld<u32x4>(sC, i * kPrepStride + q * 16);
    }
    for (int idx = tid; idx < kN * kQ / 8; idx += kPrepThreads) {
        const int n = idx >> 3, jq = idx & 7;
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = lds_ld<uint16_t>(sB, (8 * jq + 2 * e) * kPrepStride + n * 2);
            const uint32_t hi = lds_ld<uint16_t>(sB, (8 * jq + 2 * e + 1) * kPrepStride + n * 2);
            w4[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(wsBt + unit * kWsBt + n * kQ + jq * 8) =
            u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
    // G = C B^T with the causal mask applied (G[i][j] = 0 for j > i), all 16 tiles written;
    // wave w owns the tile of rows 16 (w % 4) .. +15 and columns 16 (w / 4) .. +15
    const int lane = tid & 63, li = lane & 15, g4 = lane >> 4;
    const int wave = (tid >> 6) & 3;
    static_assert(kPrepThreads == 16 * 64, "sixteen waves");
    {
        const int jt = tid >> 8;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (jt <= wave) {
#pragma unroll
            for (int m = 0; m < kN / 32; ++m) {
                const bf16x8 av = lds_ld<bf16x8>(sC, (16 * wave + li) * kPrepStride + (32 * m + 8 * g4) * 2);
                const bf16x8 bv = lds_ld<bf16x8>(sB, (16 * jt + li) * kPrepStride + (32 * m + 8 * g4) * 2);
                acc = mfma(av, bv, acc);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * wave + 4 * g4 + r, j = 16 * jt + li;
            wsG[unit * kWsG + i * kQ + j] = j <= i ? acc[r] : 0.0f;
        }
    }
}

// =======================================================================================
// main kernel
// =======================================================================================
// LDS, all tiles stored as rows of 16-byte pieces under XOR swizzles chosen so that every 8
// consecutive lanes of a ds_read_b128 / ds_write_b128 (the lanes one 128-byte LDS cycle
// serves) touch 8 different 16-byte bank groups.  Three separate arrays: the two that the
// producers fill by memory-to-LDS transfers (tiles, raw x rows) and the rest, so that the
// compiler orders an LDS access after an outstanding transfer only when it may touch the
// transfer's array.
//   tile stage s (two, by chunk parity), loaded one chunk ahead of its use:
constexpr int kCbC = 0;                          // C   [64 tok][16 pieces], piece ^ (tok & 15)
constexpr int kCbBt = kCbC + kQ * 256;           // B^T [128 n][8 pieces], piece ^ bt_swz(n)
constexpr int kCbBytes = kCbBt + kN * 128;
//   M stage s (two, by chunk parity), produced one chunk ahead of its use:
// M: only j <= i is used, so rows 0-31 hold pieces 0-3 (64 bytes) and rows 32-63 all eight
// (128 bytes): 6 KB each for hi and lo (see sw_m)
constexpr int kMBytes = 32 * 64 + 32 * 128;
constexpr int kStMhi = 0;
constexpr int kStMlo = kStMhi + kMBytes;
constexpr int kStageBytes = kStMlo + kMBytes;
//   scalar stage (three, by chunk index mod 3), produced two chunks ahead of its use: in the
//   iteration that contracts chunk c, the consumers read chunk c's E / W / decay, the
//   producers build chunk c+1's M tiles from its cum / R / r, and write chunk c+2's scalars
constexpr int kScCum = 0;                        // cum2_j = log2(e) sum_{tau<=j} dt_tau A
constexpr int kScDt = kScCum + kQ * 4;           // dt_j
constexpr int kScR = kScDt + kQ * 4;             // r_j, the last reset <= j (-1: none)
constexpr int kScRf = kScR + kQ * 4;             // R_j = 2^(cum2_{j&~7} - cum2_j) dt_j
constexpr int kScE = kScRf + kQ * 4;             // E_i = exp(cum_i) on the leading segment
constexpr int kScW = kScE + kQ * 4;              // W_j = exp(cum_last - cum_j) dt_j
constexpr int kScDecay = kScW + kQ * 4;          // exp(cum_last) (0 after a reset), 4 copies
constexpr int kScFactored = kScDecay + 16;       // 1 when the factored M exponentials apply
constexpr int kScBytes = kScFactored + 16;
//   raw x slot (three, by chunk index mod 3), loaded two chunks ahead: the conv of chunk c+1
//   runs while chunk c is contracted, and chunk c's rows stay for the consumers' exact
//   recomputation of the conv outputs the fast path flagged
constexpr int kRowsMax = kQ + kKmax - 1;         // raw x rows of a chunk incl. the conv halo
constexpr int kRwX = 0;                          // raw x [rows][8 pieces], piece ^ xr_swz(row)
constexpr int kRwSeq = (kRowsMax + 1) * 128;     // seq ids of the raw rows (after 72 row slots:
                                                 // the loads fill 9 blocks of 8 rows)
constexpr int kRwClean = kRwSeq + 72 * 4;        // bit r: run r's taps carry one id (see clean_runs)
constexpr int kRawBytes = kRwClean + 16;
//   X slot (two, by chunk parity): the conv waves' bf16 outputs (X operands), 16 bytes per
//   (wave, lane, run), read back by the consumer lane with the same wave-in-role and lane index
constexpr int kXBytes = kQ * kP * 2;
//   flag slot (two, by chunk parity): per X slot lane, one 16-bit mask per 8-output run of
//   the outputs the conv's fast path could not round with certainty
constexpr int kFlBytes = 4 * 64 * 4;
constexpr int kOffSc = 0;
constexpr int kOffX = kOffSc + 3 * kScBytes;
constexpr int kOffFl = kOffX + 2 * kXBytes;
//   conv weights and bias of the head's x channels in double (with a conv), for the out-of-line
//   recomputations (flagged outputs, masked runs): channel p at kOffW + p * kWStride
constexpr int kWStride = (kKmax + 1) * 8;
constexpr int kOffW = kOffFl + 2 * kFlBytes;
constexpr int kMainLds = kOffW + kP * kWStride;
static_assert(kMainLds + 2 * kStageBytes + 2 * kCbBytes + 3 * kRawBytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int sw_c(int tok, int q) { return tok * 256 + ((q ^ (tok & 15)) << 4); }
// B^T rows are read through the state-tile row map n = 32T + 8(l>>2) + 4(t&1) + (l&3):
// bits 0-1 and 3 of n differ across 8 consecutive lanes
__device__ __forceinline__ int sw_bt(int n, int q) {
    return n * 128 + ((q ^ ((n & 3) | (((n >> 3) & 1) << 2))) << 4);
}
// byte offset of 16-byte piece q (8 bf16 columns) of M row `row`; rows below 32 have pieces
// 0-3 only.  The swizzles keep a 16-row x 16-byte MFMA operand read at two lanes per bank
// group (the minimum for 256 bytes per 16 lanes).
__device__ __forceinline__ int sw_m(int row, int q) {
    return row < 32 ? row * 64 + ((q ^ ((row >> 1) & 3)) << 4)
                    : 32 * 64 + (row - 32) * 128 + ((q ^ (row & 7)) << 4);
}
// raw x rows: the consumers' 2-byte reads hit rows 8 apart in the four 16-lane groups
__device__ __forceinline__ int sw_xr(int row, int q) {
    return row * 128 + ((q ^ (((row >> 3) & 3) << 1)) << 4);
}

// M is built in 16 x 16 blocks (row block I, column block J <= I: ten blocks cover j <= i);
// the consumers read it as six 16 x 32 MFMA operands, whose two blocks above the diagonal,
// (0, 1) and (2, 3), stay zero (written once).  Each producer wave pw (uniform) builds three
// blocks, slot s; waves 2 and 3 have two blocks each and build one of them twice
// (identical values to identical addresses), which keeps the code free of branches.
//   pw 0: (0,0) (1,0) (1,1)   pw 1: (2,0) (2,1) (2,2)   pw 2: (3,0) (3,1) (3,0)
//   pw 3: (3,2) (3,3) (3,2)
//   (two bits per entry, entry 3 pw + s)
__device__ __forceinline__ int blk_I(int pw, int s) { return (0xFFFA94u >> (2 * (3 * pw + s))) & 3; }
__device__ __forceinline__ int blk_J(int pw, int s) { return (0xB84910u >> (2 * (3 * pw + s))) & 3; }

// Raw buffer resource over [base, base + bytes): loads past the end return 0 and stores past
// it are dropped by the hardware range check, which handles the ragged last chunk.
typedef __amdgpu_buffer_rsrc_t Rsrc;
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): wait until at most 0 / 2 vector-memory operations are outstanding
constexpr int kWaitVm0 = 0x0F70;
// vector-memory loads of the producer's registers (fetch_g, fetch_s) per iteration
template <bool HAS_SEQ, int PASS>
constexpr int reg_loads() { return (PASS == 0 ? 3 : 0) + 1 + (HAS_SEQ ? 2 : 0); }
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFFLL ? 0x7FFFFFFFLL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                             0x00020000);
}
__device__ __forceinline__ u32x4 bload128(Rsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload32(Rsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Per-block bases; everything inside one (row, head) is addressed with 32-bit offsets
// (the host checks that seqlen * channels fits).
struct Blk {
    const uint16_t* x;      // x channel 0 of this head at token 0 of this row
    const float* dt;        // dt of this head at token 0 of this row
    const int32_t* seq;     // seq_idx of this row, or NULL
    uint16_t* y;            // y channel 0 of this head at token 0 of this row
    const uint16_t* wsC;    // workspace tiles of (this row, chunk 0, this group)
    const uint16_t* wsBt;
    const float* wsG;
    int64_t ws_step;        // elements between consecutive chunks' tiles (G units)
    int L, x_row, H;
};

// Per-lane constant byte offsets of the producer's loads and stores.  The C, B^T and raw x
// tiles go straight from memory into LDS (buffer loads with the lds modifier): one
// instruction moves 64 x 16 bytes to 1 KB of consecutive LDS, lane l at byte 16 l, so each
// lane loads the global piece that the LDS swizzle puts in its slot.
struct POff {
    uint32_t c[4];          // C tile LDS block r = 4 pw + k: token 4r + l/16, slot l%16
    uint32_t bt[4];         // B^T tile LDS block r = 4 pw + k: row n = 8r + l/8, slot l%8
    uint32_t x[3];          // raw x LDS blocks r = pw, pw + 4, 8: row 8r + l/8, slot l%8
    uint32_t g[3];          // G piece of M block slot s: row i, columns 4 lanes' worth
    uint32_t dt;            // token = lane
};

// Registers a producer lane loads ahead of use: a chunk's dt and ids (its scalars, two
// chunks ahead of the contraction) and a chunk's G pieces (its M blocks, one chunk ahead)
struct FetchS {
    uint32_t dt;
    int32_t seq_j, seq_prev;
};
struct FetchG {
    u32x4 gm[3];
};

__device__ __forceinline__ void dma16(Rsrc r, uint32_t voff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Chunk k's C / B^T tiles into tile stage `st` (the state-only pass needs B^T alone)
template <int PASS>
__device__ __forceinline__ void fetch_tiles(const Blk& bk, const POff& o, int64_t k, int pw,
                                            uint8_t* st) {
    const Rsrc rc = make_rsrc(bk.wsC + k * bk.ws_step * kWsC, kWsC * 2);
    const Rsrc rb = make_rsrc(bk.wsBt + k * bk.ws_step * kWsBt, kWsBt * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (PASS == 0) dma16(rc, o.c[q], st + kCbC + (4 * pw + q) * 1024);
        dma16(rb, o.bt[q], st + kCbBt + (4 * pw + q) * 1024);
    }
}

// Chunk k's G pieces into registers (the state-only pass has no M)
template <int PASS>
__device__ __forceinline__ void fetch_g(const Blk& bk, const POff& o, int64_t k, FetchG& f) {
    if (PASS == 0) {
        const Rsrc rg = make_rsrc(bk.wsG + k * bk.ws_step * kWsG, kWsG * 4);
#pragma unroll
        for (int s = 0; s < 3; ++s) f.gm[s] = bload128(rg, o.g[s]);
    }
}

// Chunk k's dt and ids into registers; past the row's end the range check returns zeros
template <bool HAS_SEQ>
__device__ __forceinline__ void fetch_s(const Blk& bk, const POff& o, int64_t k, int lane,
                                        FetchS& f) {
    const int t0 = static_cast<int>(k) * kQ;
    const Rsrc rd = make_rsrc(bk.dt + static_cast<int64_t>(t0) * bk.H, static_cast<int64_t>(bk.L - t0) * bk.H * 4);
    f.dt = bload32(rd, o.dt);
    if (HAS_SEQ) {
        const Rsrc rs = make_rsrc(bk.seq + t0, static_cast<int64_t>(bk.L - t0) * 4);
        f.seq_j = static_cast<int32_t>(bload32(rs, lane * 4));
        f.seq_prev = bk.seq[t0 <= 0 ? 0 : (t0 <= bk.L ? t0 - 1 : bk.L - 1)];
    }
}

// With seq_idx: bit r set when raw rows 8r .. 8r+K+6 (the taps of run r, tokens 8r .. 8r+7)
// carry one sequence id.  Computed once per chunk by producer wave 0 from the ids of rows
// 0 .. 63 (id_lo, row = lane) and 64 .. K+62 (id_hi, row = 64 + lane): a boundary bit per row
// where the id differs from the row before, then one window test per run on the wave-uniform
// masks.  The conv lanes read the word instead of comparing their windows' ids themselves.
template <int K>
__device__ __forceinline__ uint32_t clean_runs(int32_t id_lo, int32_t id_hi, int lane) {
    constexpr int kRows = kQ + K - 1;
    const int32_t prev_lo = __shfl_up(id_lo, 1);
    const uint64_t b_lo = __ballot(lane >= 1 && id_lo != prev_lo);      // bit rho: rows rho-1, rho
    const int32_t last = __builtin_amdgcn_readlane(id_lo, kQ - 1);
    int32_t prev_hi = __shfl_up(id_hi, 1);
    if (lane == 0) prev_hi = last;
    const uint64_t b_hi = __ballot(lane < kRows - kQ && id_hi != prev_hi);  // bit l: row 64 + l
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < kQ / 8; ++r) {
        const int j0 = 8 * r;  // boundaries that matter: rows j0+1 .. j0+K+6
        const uint64_t w = (b_lo >> (j0 + 1)) | (b_hi << (kQ - 1 - j0));
        if ((w & ((1ull << (K + 6)) - 1)) == 0) m |= 1u << r;
    }
    return m;
}

// Raw x rows of chunk k >= 1 (first row t0 - (K-1) >= 0) into raw slot `raw`; rows past the
// end arrive as zeros, and all of them when `live` is false.  Every wave loads LDS blocks pw
// and pw + 4 (rows 0-63) and block 8 (rows 64-71, the same data from every wave), with no
// branch.  With seq_idx the rows' ids come back in *seq_row, to be stored once the load has
// landed.
template <int K, bool HAS_SEQ>
__device__ __forceinline__ void fetch_raw(const Blk& bk, const POff& o, int64_t k, bool live,
                                          int pw, int lane, uint8_t* raw, int32_t* seq_row,
                                          int32_t* seq_hi) {
    constexpr int kRows = kQ + K - 1;
    const int r0 = live ? static_cast<int>(k) * kQ - (K - 1) : 0;
    const Rsrc rx = make_rsrc(bk.x + static_cast<int64_t>(r0) * bk.x_row,
                              live ? static_cast<int64_t>(bk.L - r0) * bk.x_row * 2 : 0);
    dma16(rx, o.x[0], raw + kRwX + pw * 1024);
    dma16(rx, o.x[1], raw + kRwX + (pw + 4) * 1024);
    dma16(rx, o.x[2], raw + kRwX + 8 * 1024);
    if (HAS_SEQ) {
        const int ptid = pw * 64 + lane;
        const Rsrc rs = make_rsrc(bk.seq + r0, live ? static_cast<int64_t>(bk.L - r0) * 4 : 0);
        if (ptid < kRows) *seq_row = static_cast<int32_t>(bload32(rs, ptid * 4));
        // wave 0 also takes rows 64 .. (the clean-run mask); the same values as wave 1's
        if (pw == 0 && kQ + lane < kRows) *seq_hi = static_cast<int32_t>(bload32(rs, (kQ + lane) * 4));
    }
}

// raw x rows of a block's first chunk (first token t0; rows before token 0 come from the
// conv state), straight to LDS
template <int K, bool FUSED, bool HAS_SEQ>
__device__ __forceinline__ void stage_raw_first(const ChunkedArgs& a, const Blk& bk, int64_t b,
                                                int64_t h, int t0, int pw, int lane, uint8_t* raw) {
    constexpr int kRows = kQ + K - 1;
    const int ptid = pw * 64 + lane;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int idx = ptid + 256 * k;
        if (idx < kRows * 8) {
            const int rho = idx >> 3, q = idx & 7;
            const int t = t0 + rho - (K - 1);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t >= 0 && t < bk.L) {
                v = *reinterpret_cast<const u32x4*>(bk.x + static_cast<int64_t>(t) * bk.x_row + q * 8);
            } else if (FUSED && t < 0 && a.conv_init) {
                const int64_t cc0 = a.x_col0 + h * kP + q * 8;
                uint32_t w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = a.conv_init[(b * a.C_conv + cc0 + 2 * e) * (K - 1) + (K - 1) + t];
                    const uint32_t hi = a.conv_init[(b * a.C_conv + cc0 + 2 * e + 1) * (K - 1) + (K - 1) + t];
                    w4[e] = lo | (hi << 16);
                }
                v = u32x4{w4[0], w4[1], w4[2], w4[3]};
            }
            lds_st(raw, kRwX + sw_xr(rho, q), v);
        }
    }
    if (HAS_SEQ) {
        auto id_of = [&](int rho) {
            int tr = t0 + rho - (K - 1);
            tr = tr < 0 ? 0 : (tr >= bk.L ? bk.L - 1 : tr);
            return bk.seq[tr];
        };
        if (ptid < kRows) reinterpret_cast<int32_t*>(raw + kRwSeq)[ptid] = id_of(ptid);
        if (pw == 0) {
            const uint32_t m = clean_runs<K>(id_of(lane), kQ + lane < kRows ? id_of(kQ + lane) : 0, lane);
            if (lane == 0) *reinterpret_cast<uint32_t*>(raw + kRwClean) = m;
        }
    }
}

// Chunk k's scalars from its fetched dt / ids, into scalar stage `sc` (every producer wave
// computes and writes the same values, which keeps the code free of branches):
//   cum2_j = log2(e) * sum_{tau<=j} dt_tau A (wave prefix scan), r_j = last reset <= j,
//   E_i = 2^cum2_i, W_j = 2^(cum2_last - cum2_j) dt_j, decay = 2^cum2_last,
//   R_j = 2^(cum2_{j0} - cum2_j) dt_j with j0 = j & ~7 (the column factor of M, below).
// The factored form of M's exponentials holds when cum2 never increases within the chunk and
// each 8-column group spans at most 64 (then R_j <= 2^64 dt_j and the row factor <= 1 on and
// below the diagonal); otherwise the M blocks take one exponential per entry.
template <bool HAS_SEQ, int PASS>
__device__ __forceinline__ void chunk_scalars(const FetchS& f, int64_t k, int L, float Ah2,
                                              int lane, uint8_t* sc) {
    const int t0 = static_cast<int>(k) * kQ;
    const int j = lane;
    const float dtv = __uint_as_float(f.dt);
    const float a2 = dtv * Ah2;
    const float cum = wave_incl_sum(a2);
    int r = -1;
    if (HAS_SEQ) {
        int32_t sjm1 = __shfl_up(f.seq_j, 1);
        if (lane == 0) sjm1 = f.seq_prev;
        const int rst = (t0 + j < L && t0 + j > 0 && f.seq_j != sjm1) ? j : -1;
        r = wave_incl_max(rst);
    }
    const float cum_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), kQ - 1));
    const int r_last = HAS_SEQ ? __builtin_amdgcn_readlane(r, kQ - 1) : -1;
    reinterpret_cast<float*>(sc + kScE)[j] = r < 0 ? __builtin_amdgcn_exp2f(cum) : 0.0f;
    reinterpret_cast<float*>(sc + kScW)[j] = j >= r_last ? __builtin_amdgcn_exp2f(cum_last - cum) * dtv : 0.0f;
    // decay slot: lanes 0-3 write 4 copies; consumers read copy 0
    reinterpret_cast<float*>(sc + kScDecay)[j & 3] = r_last < 0 ? __builtin_amdgcn_exp2f(cum_last) : 0.0f;
    if (PASS == 1) return;  // the state-only pass needs W and the decay alone
    reinterpret_cast<float*>(sc + kScCum)[j] = cum;
    reinterpret_cast<float*>(sc + kScDt)[j] = dtv;
    if (HAS_SEQ) reinterpret_cast<int32_t*>(sc + kScR)[j] = r;
    // cum2 of the group's first column from lane j & ~7 (swizzle within 32-lane halves:
    // and-mask 0x18)
    const float cg = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(cum), 0x0018));
    const float span = cg - cum;
    reinterpret_cast<float*>(sc + kScRf)[j] = __builtin_amdgcn_exp2f(span) * dtv;
    const bool factored = __ballot(!(a2 <= 0.0f && span <= 64.0f)) == 0;  // NaN -> direct
    reinterpret_cast<int32_t*>(sc + kScFactored)[j & 3] = factored ? 1 : 0;
}

// This wave's three 16 x 16 blocks of chunk k's M = G o 2^(cum2_i - cum2_j) dt_j on
// r_i <= j <= i (G is 0 above the diagonal), from the chunk's scalar stage `sc` (written in an
// earlier iteration) and the G pieces fetched for it, split hi / lo (MBlk, stored into an M
// stage by store_m).  A lane holds row i = 16 I + l % 16 and columns j0 .. j0+3,
// j0 = 16 J + 4 (l / 16); these share the 8-column group of j0 & ~7, so the exponential
// splits into the row factor 2^(cum2_i - cum2_{j0 & ~7}) (one per lane) times the column
// factors R_j.
struct MBlk {
    u32x2 hi[3], lo[3];
};
template <bool HAS_SEQ>
__device__ __forceinline__ void m_blocks(const FetchG& f, int pw, int lane, const uint8_t* sc,
                                         MBlk& mb) {
    const bool factored = __builtin_amdgcn_readfirstlane(lds_ld<int32_t>(sc, kScFactored)) != 0;
    float mv[3][4];
    if (factored) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int i = 16 * blk_I(pw, s) + (lane & 15), j0 = 16 * blk_J(pw, s) + 4 * (lane >> 4);
            const float prow = __builtin_amdgcn_exp2f(lds_ld<float>(sc, kScCum + i * 4) -
                                                      lds_ld<float>(sc, kScCum + (j0 & ~7) * 4));
            const f32x4 rj = lds_ld<f32x4>(sc, kScRf + j0 * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) mv[s][e] = __uint_as_float(f.gm[s][e]) * rj[e] * prow;
        }
    } else {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int i = 16 * blk_I(pw, s) + (lane & 15), j0 = 16 * blk_J(pw, s) + 4 * (lane >> 4);
            const float ci = lds_ld<float>(sc, kScCum + i * 4);
            const f32x4 cj = lds_ld<f32x4>(sc, kScCum + j0 * 4);
            const f32x4 dj = lds_ld<f32x4>(sc, kScDt + j0 * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mv[s][e] = __uint_as_float(f.gm[s][e]) * __builtin_amdgcn_exp2f(ci - cj[e]) * dj[e];
        }
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int i = 16 * blk_I(pw, s) + (lane & 15), j0 = 16 * blk_J(pw, s) + 4 * (lane >> 4);
        const int ri = HAS_SEQ ? lds_ld<int32_t>(sc, kScR + i * 4) : -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float m = mv[s][e];
            m = j0 + e <= i ? m : 0.0f;   // overflow / 0 * inf above the diagonal
            if (HAS_SEQ) m = j0 + e >= ri ? m : 0.0f;
            mv[s][e] = m;
        }
        split_hilo4(mv[s], mb.hi[s], mb.lo[s]);
    }
}
__device__ __forceinline__ void store_m(const MBlk& mb, int pw, int lane, uint8_t* st) {
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int i = 16 * blk_I(pw, s) + (lane & 15), j0 = 16 * blk_J(pw, s) + 4 * (lane >> 4);
        const int off = sw_m(i, j0 >> 3) + (j0 & 4) * 2;
        lds_st(st, kStMhi + off, mb.hi[s]);
        lds_st(st, kStMlo + off, mb.lo[s]);
    }
}

// Consumer: the conv of channel p over tokens j0 .. j0+7 of a chunk from its staged raw rows
// (row rho <-> token t0 - (K-1) + rho), rounded to bf16 -> one MFMA operand.  MODE 0: no conv
// (the rows already hold x); 1: conv, identity phi; 2: conv + SiLU.  The fast path has no
// branches, so the scheduler can spread it between the contractions of the previous chunk;
// for SiLU it flags, in *near, outputs that lie too close to a bf16 rounding midpoint for
// the fp32 evaluation to decide (conv_fixups redoes those in double).
template <int K, int MODE, bool HAS_SEQ>
__device__ __forceinline__ double conv_z(const uint8_t* raw, int q, int byte, int r0,
                                         const double (&cw)[K], double cbias) {
    double z = cbias;
    int32_t idl = 0;
    if (HAS_SEQ) idl = lds_ld<int32_t>(raw, kRwSeq + (r0 + K - 1) * 4);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        double u = bf16_to_f32(lds_ld<uint16_t>(raw, kRwX + sw_xr(r0 + k, q) + byte));
        if (HAS_SEQ && lds_ld<int32_t>(raw, kRwSeq + (r0 + k) * 4) != idl) u = 0.0;
        z = fma(cw[k], u, z);
    }
    return z;
}

template <int K, int MODE, bool HAS_SEQ>
__device__ __forceinline__ bf16x8 conv_fast(const uint8_t* raw, int p, int j0,
                                            const double (&cw)[K], double cbias, uint32_t* near) {
    bf16x8 out;
    const int q = p >> 3, byte = (p & 7) * 2;
    if (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            out[e] = __builtin_bit_cast(__bf16, lds_ld<uint16_t>(raw, kRwX + sw_xr(j0 + e + K - 1, q) + byte));
        return out;
    }
    double u[8 + K - 1];
    int32_t id[8 + K - 1];
#pragma unroll
    for (int tau = 0; tau < 8 + K - 1; ++tau) {
        u[tau] = bf16_to_f32(lds_ld<uint16_t>(raw, kRwX + sw_xr(j0 + tau, q) + byte));
        id[tau] = HAS_SEQ ? lds_ld<int32_t>(raw, kRwSeq + (j0 + tau) * 4) : 0;
    }
    float zf[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        double z = cbias;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const double tap = (!HAS_SEQ || id[e + k] == id[e + K - 1]) ? u[e + k] : 0.0;
            z = fma(cw[k], tap, z);
        }
        if (MODE == 2) {
            zf[e] = static_cast<float>(z);
            sv[e] = zf[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-zf[e]));
        } else {
            out[e] = __builtin_bit_cast(__bf16, f64_to_bf16(z));
        }
    }
    if (MODE == 2) {
        // near a bf16 rounding midpoint: the fp32 SiLU of the exactly summed z is within
        // 7 + 3|z| ulps of the exact value (see silu_f32), so an output whose low 16 bits lie
        // within 8 + 4|z| of 0x8000 cannot be rounded with certainty.  One bound per run (its
        // largest |z|, rounded up to an integer, at most 0x8000: then every output is near);
        // the test is lo16 - (0x8000 - bnd) <= 2 bnd modulo 2^16.  The per-output tests land
        // in lane masks, and only when some lane has a flagged output are they turned into
        // per-lane bits.
        float zm = fabsf(zf[0]);
#pragma unroll
        for (int e = 1; e < 8; ++e) zm = fmaxf(zm, fabsf(zf[e]));
        const uint32_t bnd = min(static_cast<uint32_t>(fmaf(4.0f, zm, 9.0f)), 0x8000u);
        const uint16_t edge = static_cast<uint16_t>(0x8000u - bnd);
        uint64_t m[8], any = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t t = static_cast<uint16_t>(static_cast<uint16_t>(__float_as_uint(sv[e])) - edge);
            m[e] = __builtin_amdgcn_ballot_w64(static_cast<uint32_t>(t) <= 2u * bnd);
            any |= m[e];
            out[e] = static_cast<__bf16>(sv[e]);
        }
        uint32_t nb = 0;
        if (any != 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) nb |= __builtin_amdgcn_inverse_ballot_w64(m[e]) ? (1u << e) : 0u;
        }
        *near = nb;   // bit e: output e
    }
    return out;
}

// Redo, in double, the SiLU outputs of one run (tokens j0 .. j0+7) that conv_fast flagged.
// Flagged outputs are rare: one branch skips everything when no lane has a flag, and each
// output's recomputation is skipped when no lane has that one.
template <int K, int MODE, bool HAS_SEQ>
__device__ __forceinline__ bf16x8 conv_fixups(const uint8_t* raw, int p, int j0,
                                              const double (&cw)[K], double cbias,
                                              uint32_t near, bf16x8 x) {
    if (MODE == 2 && near) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (near & (1u << e)) {
                const double z = conv_z<K, 2, HAS_SEQ>(raw, p >> 3, (p & 7) * 2, j0 + e, cw, cbias);
                x[e] = __builtin_bit_cast(__bf16, silu_f64_to_bf16(z));
            }
        }
    }
    return x;
}

// One conv + SiLU output (channel p, taps from raw row r0), rounded exactly, with the weights
// from the LDS table: the consumers' rare recomputation of a flagged output, out of line so
// that its double-precision registers do not count against the contraction loop
template <int K>
__device__ __noinline__ uint32_t silu_conv_exact(const uint8_t* raw, const uint8_t* wt, int p, int r0) {
    double cw[K];
#pragma unroll
    for (int k = 0; k < K; ++k) cw[k] = lds_ld<double>(wt, p * kWStride + 8 * k);
    const double cbias = lds_ld<double>(wt, p * kWStride + 8 * K);
    const double z = conv_z<K, 2, false>(raw, p >> 3, (p & 7) * 2, r0, cw, cbias);
    return silu_f64_to_bf16(z);
}

// The conv of channel p over tokens j0 .. j0+7 with the sequence masks, one output at a
// time, each written over the fast path's value at xs + off + 2e (the rare runs whose taps
// straddle a sequence boundary).  Out of line, with the weights from the LDS table: weights
// passed in as an array would go through the stack, a round trip to memory per call.
template <int K, int MODE>
__device__ __noinline__ void conv_masked_run(const uint8_t* raw, const uint8_t* wt, int p, int j0,
                                             uint8_t* xs, int off) {
    double cw[K];
#pragma unroll
    for (int k = 0; k < K; ++k) cw[k] = lds_ld<double>(wt, p * kWStride + 8 * k);
    const double cbias = lds_ld<double>(wt, p * kWStride + 8 * K);
    for (int e = 0; e < 8; ++e) {
        const double z = conv_z<K, MODE, true>(raw, p >> 3, (p & 7) * 2, j0 + e, cw, cbias);
        const uint16_t v = MODE == 2 ? act_to_bf16(z, SSM_ACT_SILU) : f64_to_bf16(z);
        *reinterpret_cast<uint16_t*>(xs + off + 2 * e) = v;
    }
}

// conv weights and bias of x channel p of head h, as doubles (zeros without a conv)
template <int K, int MODE>
__device__ __forceinline__ void conv_weights(const ChunkedArgs& a, int64_t h, int p,
                                             double (&cw)[K], double& cbias) {
    cbias = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) cw[k] = 0.0;
    if (MODE != 0) {
        const int64_t cc = a.x_col0 + h * kP + p;
#pragma unroll
        for (int k = 0; k < K; ++k) cw[k] = a.conv_w[cc * K + k];
        cbias = a.conv_b ? a.conv_b[cc] : 0.0f;
    }
}

// PASS 0: the full scan of a block's chunks.  PASS 1 (long rows split into segments): the
// end state of every segment but the last from a zero start, and its decay product.
template <int K, int MODE, bool HAS_SEQ, int PASS>
__global__ void __launch_bounds__(kMainThreads, 1)
ssd_main_kernel(ChunkedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[kMainLds];
    // the M stages are an array of their own: the compiler then orders the producers' M
    // stores after an outstanding memory-to-LDS transfer only when they may overlap
    __shared__ __attribute__((aligned(16))) uint8_t sm_m[2 * kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sm_cb[2 * kCbBytes];
    // raw slots 0 and 1 are separate arrays, so the compiler can tell a load into one slot
    // from reads of the other
    __shared__ __attribute__((aligned(16))) uint8_t sm_raw0[kRawBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sm_raw1[kRawBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sm_raw2[kRawBytes];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, li = lane & 15, g4 = lane >> 4;
    const int role = wave >> 2;  // 0 consumer, 1 producer, 2 conv

    // block -> (row, segment, head): consecutive units on one XCD (blocks are dealt round-robin
    // over the 8 XCDs), so the heads of one row segment share that XCD's L2 for the B/C/G tiles
    const int64_t nsl = PASS == 1 ? a.nseg - 1 : a.nseg;
    const int64_t nblk = gridDim.x;
    const int64_t kb = blockIdx.x;
    const int64_t u = (nblk % 8 == 0) ? (kb % 8) * (nblk / 8) + kb / 8 : kb;
    const int64_t h = u % a.H, bsg = u / a.H;
    const int64_t b = bsg / nsl, seg = bsg % nsl;
    const int64_t g = h / (a.H / a.G);
    const int64_t L = a.L;
    const int64_t nC = (L + kQ - 1) / kQ;
    // the row of the initial / final state arrays this batch row uses
    const int64_t srow = a.state_slots ? static_cast<int64_t>(a.state_slots[b]) : b;
    const bool srow_ok = a.n_state_slots <= 0 || (srow >= 0 && srow < a.n_state_slots);
    // this block's chunks: global chunk c0 + c for c < nCl
    int64_t c0 = seg * a.seg_chunks;
    int64_t nCl = min(a.seg_chunks, nC - c0);
    const float Ah = a.A[h];
    // the state-only pass starts where the earlier chunks can no longer reach the end state
    bool skipped = false;
    if constexpr (PASS == 1) {
        const int64_t skip = state_pass_skip<kMainThreads>(a.dt + b * L * a.H + h, a.H, L, c0, nCl,
                                                           Ah, reinterpret_cast<float*>(sm), tid);
        c0 += skip;
        nCl -= skip;
        skipped = skip > 0;
    }
    Blk bk;
    bk.x = a.x + b * L * a.x_row + a.x_col0 + h * kP;
    bk.dt = a.dt + b * L * a.H + h;
    bk.seq = a.seq_idx ? a.seq_idx + b * L : nullptr;
    bk.y = a.y + (b * L * a.H + h) * kP;
    {
        const uint16_t* ws = static_cast<const uint16_t*>(a.workspace);
        const int64_t units = a.B * nC * a.G;
        const int64_t unit0 = ws_unit(a, b, 0, g, nC);
        bk.wsC = ws + unit0 * kWsC;
        bk.wsBt = ws + units * kWsC + unit0 * kWsBt;
        bk.wsG = reinterpret_cast<const float*>(ws + units * (kWsC + kWsBt)) + unit0 * kWsG;
        bk.ws_step = a.G;
    }
    bk.L = static_cast<int>(L);
    bk.x_row = static_cast<int>(a.x_row);
    bk.H = static_cast<int>(a.H);

    // The three roles run separate loops (a wave's role never changes), so the register
    // allocator sees each role's live ranges alone, and each SIMD holds one wave of each role
    // to interleave.  All loops pass the same number of block barriers: three in the prologue
    // (raw rows of chunk 0 staged; scalars of chunks 0 and 1 written; chunk 0 produced and
    // convolved), then one per chunk.
    // Between two barriers:
    //   consumers  contract chunk c from M stage c&1, scalar stage c%3 and X slot c&1 and
    //              store y(c);
    //   producers  load chunk c+1's tiles into tile stage (c+1)&1 and chunk c+2's raw rows
    //              into raw slot (c+2)%3, compute chunk c+2's scalars and chunk c+1's M
    //              blocks, then load the registers those need one iteration later;
    //   conv waves convolve chunk c+1 from raw slot (c+1)%3 into X slot (c+1)&1.
    if (role == 0) {
        // state slice acc[t][r] = h[p][n], p = 16 wave + li, n = 32(t/2) + 8 g4 + 4(t%2) + r
        // (the MFMA row of tile t that lane group g4 holds)
        const int p_own = 16 * wave + li;
        f32x4 acc[8];
        {
            // Row segments keep their states in the slots seg_state[b, h, s]: slot 0 the
            // initial state (copied there by segment 0's state-only block, so the full pass
            // never reads initial_state, which an in-place final state may overwrite), slot
            // s >= 1 segment s-1's local end state l_{s-1}.  A full-pass block composes its
            // entry state e_seg in order: e_0 = slot 0, e_s = D_{s-1} e_{s-1} + l_{s-1} ([LG]
            // Sec. 2.5's initial-state increment, applied segment by segment).
            const float* init =
                a.init_state && srow_ok ? a.init_state + ((srow * a.H + h) * kP + p_own) * kN : nullptr;
            float* slots = a.nseg > 1 ? a.seg_state + ((b * a.H + h) * a.nseg * kP + p_own) * kN : nullptr;
            const float* src = PASS == 1 ? (seg == 0 ? init : nullptr) : (a.nseg > 1 ? slots : init);
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
            if (PASS == 1) {
                if (seg == 0) {
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        *reinterpret_cast<f32x4*>(slots + 32 * m + 8 * g4) = acc[2 * m];
                        *reinterpret_cast<f32x4*>(slots + 32 * m + 8 * g4 + 4) = acc[2 * m + 1];
                    }
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            } else if (a.nseg > 1) {
                for (int64_t sg = 1; sg <= seg; ++sg) {
                    const float d = a.seg_decay[(b * a.H + h) * a.nseg + sg - 1];
                    const float* ls = slots + sg * (kP * kN);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        acc[2 * m] = d * acc[2 * m] + *reinterpret_cast<const f32x4*>(ls + 32 * m + 8 * g4);
                        acc[2 * m + 1] = d * acc[2 * m + 1] + *reinterpret_cast<const f32x4*>(ls + 32 * m + 8 * g4 + 4);
                    }
                }
            }
        }
        __syncthreads();  // raw rows of chunk 0 staged
        __syncthreads();  // scalars of chunks 0 and 1 written
        __syncthreads();  // stage 0 and X(0) ready
        // X operands (lane: channel p_own, tokens 32 s + 8 g4 .. +7), convolved by the conv
        // wave with this wave's index
        const int xoff = (wave * 64 + lane) * 32;
        // y: bytes between tokens, and this lane's offset from the chunk's first token row
        const uint32_t y_tok = static_cast<uint32_t>(bk.H) * kP * 2;
        const uint32_t y_off = li * y_tok + (16 * wave + 4 * g4) * 2;
        float dprod = 1.0f;  // decay product of the block's chunks (state-only pass)
        int rslot = 0;  // raw slot of chunk cn
        for (int64_t cn = 0; cn < nCl; ++cn) {
            const uint8_t* st = sm_m + (cn & 1) * kStageBytes;
            const uint8_t* sc = sm + kOffSc + rslot * kScBytes;  // scalar stage cn % 3
            const uint8_t* cbt = sm_cb + (cn & 1) * kCbBytes;
            bf16x8 xv[2];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) xv[sh] = lds_ld<bf16x8>(sm + kOffX + (cn & 1) * kXBytes, xoff + 16 * sh);
            uint32_t flw = 0;  // bit 16 sh + e: output e of xv[sh] needs the exact recomputation
            if constexpr (MODE == 2) flw = lds_ld<uint32_t>(sm + kOffFl + (cn & 1) * kFlBytes, (wave * 64 + lane) * 4);

            // Y^T[p][i], p = 16 wave + 4 g4 + r, i = 16 I + li.  Each phase loads its LDS
            // operands before its MFMAs, and consecutive MFMAs use different accumulators
            // (all hi products, then all lo products), so neither LDS latency nor the MFMA
            // result latency sits between two issues.
            // one accumulator per row block: Y_off, then scaled by E_i, then the intra-chunk
            // products on top
            f32x4 ya[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) ya[I] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const float decay = lds_ld<float>(sc, kScDecay);
            if constexpr (PASS == 0) {
            // initial-state part first (it does not need X), one 32-wide slice m of the state
            // at a time; the next slice's C tiles load while this slice's MFMAs run.  The
            // decayed state goes to new registers first, so the split may overwrite the old
            // values in place (no copies for the lo parts).
            bf16x8 cb[2][4];
#pragma unroll
            for (int I = 0; I < 4; ++I) cb[0][I] = lds_ld<bf16x8>(cbt, kCbC + sw_c(16 * I + li, g4));
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m + 1 < 4) {
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        cb[(m + 1) & 1][I] = lds_ld<bf16x8>(cbt, kCbC + sw_c(16 * I + li, 4 * (m + 1) + g4));
                }
                float hv[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hv[e] = acc[2 * m][e];
                    hv[4 + e] = acc[2 * m + 1][e];
                }
                acc[2 * m] *= decay;
                acc[2 * m + 1] *= decay;
                // the split after the decay products (an empty statement that reads them):
                // then it is the old values' last use and may overwrite them in place
#pragma unroll
                for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(hv[e]) : "v"(acc[2 * m + (e >> 2)][e & 3]));
                bf16x8 hhi, hlo;
                split_hilo(hv, hhi, hlo);
#pragma unroll
                for (int I = 0; I < 4; ++I) ya[I] = mfma(hhi, cb[m & 1][I], ya[I]);
#pragma unroll
                for (int I = 0; I < 4; ++I) ya[I] = mfma(hlo, cb[m & 1][I], ya[I]);
            }
            }
            if constexpr (MODE == 2) {
                // the conv outputs of this lane that the fast path flagged (rare): redone in
                // double from the chunk's raw rows, which stay in their slot until the chunk
                // ends, while the matrix cores work through the products above
                if (flw != 0) {
                    const uint8_t* rawc = rslot == 0 ? sm_raw0 : rslot == 1 ? sm_raw1 : sm_raw2;
                    u32x4 xw[2] = {__builtin_bit_cast(u32x4, xv[0]), __builtin_bit_cast(u32x4, xv[1])};
                    do {
                        const int bit = __builtin_ctz(flw);
                        flw &= flw - 1;
                        const int sh = bit >> 4, e = bit & 7;
                        const uint32_t v = silu_conv_exact<K>(rawc, sm + kOffW, p_own, 8 * g4 + 32 * sh + e);
                        const int word = e >> 1, shift = 16 * (e & 1);
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int d = 0; d < 4; ++d)
                                if (t == sh && d == word)
                                    xw[t][d] = (xw[t][d] & ~(0xFFFFu << shift)) | (v << shift);
                    } while (flw != 0);
                    xv[0] = __builtin_bit_cast(bf16x8, xw[0]);
                    xv[1] = __builtin_bit_cast(bf16x8, xw[1]);
                }
            }
            rslot = rslot == 2 ? 0 : rslot + 1;
            if constexpr (PASS == 0) {
            // intra-chunk part: M tiles (I, s) with 32 s <= 16 I + 15; the hi tiles, then the
            // lo tiles in the same registers (keeps the wave's peak register count down).  The
            // M tiles load while Y_off is scaled by E_i (row i = 16 I + li of the lane).
            bf16x8 mt[6];
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int I = u < 2 ? u : (u < 4 ? 2 : 3), sh = u < 2 ? 0 : ((u & 1) ? 1 : 0);
                mt[u] = lds_ld<bf16x8>(st, kStMhi + sw_m(16 * I + li, 4 * sh + g4));
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) ya[I] *= lds_ld<float>(sc, kScE + (16 * I + li) * 4);
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int I = u < 2 ? u : (u < 4 ? 2 : 3), sh = u < 2 ? 0 : ((u & 1) ? 1 : 0);
                ya[I] = mfma(xv[sh], mt[u], ya[I]);
            }
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int I = u < 2 ? u : (u < 4 ? 2 : 3), sh = u < 2 ? 0 : ((u & 1) ? 1 : 0);
                mt[u] = lds_ld<bf16x8>(st, kStMlo + sw_m(16 * I + li, 4 * sh + g4));
            }
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int I = u < 2 ? u : (u < 4 ? 2 : 3), sh = u < 2 ? 0 : ((u & 1) ? 1 : 0);
                ya[I] = mfma(xv[sh], mt[u], ya[I]);
            }
            }
            // state update: h^T[n][p] = decay h^T + B^T (W o X) (the decay is applied above
            // in the full pass)
            if constexpr (PASS == 1) {
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] *= decay;
            }
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
                float wj[8];
                {
                    const f32x4 w0 = lds_ld<f32x4>(sc, kScW + (32 * sh + 8 * g4) * 4);
                    const f32x4 w1 = lds_ld<f32x4>(sc, kScW + (32 * sh + 8 * g4 + 4) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { wj[e] = w0[e]; wj[4 + e] = w1[e]; }
                }
                bf16x8 bv[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int n_row = 32 * (t >> 1) + 8 * (li >> 2) + 4 * (t & 1) + (li & 3);
                    bv[t] = lds_ld<bf16x8>(cbt, kCbBt + sw_bt(n_row, 4 * sh + g4));
                }
                float wx[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) wx[e] = wj[e] * static_cast<float>(xv[sh][e]);
                bf16x8 bh, bl;
                split_hilo(wx, bh, bl);
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] = mfma(bv[t], bh, acc[t]);
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] = mfma(bv[t], bl, acc[t]);
            }
            if constexpr (PASS == 0) {
                // y of this chunk straight to memory: a lane stores 4 channels of token
                // 16 I + li (8 bytes), the four waves fill each 128-byte token row; rows past
                // the end of the row are dropped by the range check
                const int t0 = static_cast<int>(c0 + cn) * kQ;
                const Rsrc ry = make_rsrc(bk.y + static_cast<int64_t>(t0) * bk.H * kP,
                                          static_cast<int64_t>(bk.L - t0) * bk.H * kP * 2);
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    u32x2 pk;
                    pk[0] = pack_bf16x2(ya[I][0], ya[I][1]);
                    pk[1] = pack_bf16x2(ya[I][2], ya[I][3]);
                    __builtin_amdgcn_raw_buffer_store_b64(pk, ry, y_off + 16 * I * y_tok, 0, 0);
                }
            } else {
                dprod *= decay;
            }
            __syncthreads();
        }
        // end state: a segment's local end state goes to slot seg + 1 (the full pass of the
        // later segments composes its entry state from it); the last segment (or the only
        // one) writes the final state
        float* dst = nullptr;
        if (PASS == 1)
            dst = a.seg_state + (((b * a.H + h) * a.nseg + seg + 1) * kP + p_own) * kN;
        else if (a.final_state && srow_ok && seg == a.nseg - 1)
            dst = a.final_state + ((srow * a.H + h) * kP + p_own) * kN;
        if (dst) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                *reinterpret_cast<f32x4*>(dst + 32 * m + 8 * g4) = acc[2 * m];
                *reinterpret_cast<f32x4*>(dst + 32 * m + 8 * g4 + 4) = acc[2 * m + 1];
            }
        }
        // a skipped start means the decay product over the segment is below 1e-90: 0 in fp32
        if (PASS == 1 && wave == 0 && lane == 0)
            a.seg_decay[(b * a.H + h) * a.nseg + seg] = skipped ? 0.0f : dprod;
    } else if (role == 1) {
        const int pw = __builtin_amdgcn_readfirstlane(wave - 4);
        const float Ah2 = Ah * 1.4426950408889634f;  // exponents in base 2
        POff o;
        {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 4 * pw + q;
                const int tok = 4 * r + (lane >> 4), slot = lane & 15;
                o.c[q] = tok * 256 + ((slot ^ (tok & 15)) << 4);
                const int n = 8 * r + (lane >> 3), sl = lane & 7;
                o.bt[q] = n * 128 + ((sl ^ ((n & 3) | (((n >> 3) & 1) << 2))) << 4);
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int blk = q < 2 ? pw + 4 * q : 8;
                const int row = 8 * blk + (lane >> 3), sl = lane & 7;
                o.x[q] = row * bk.x_row * 2 + ((sl ^ (((row >> 3) & 3) << 1)) << 4);
            }
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const int i = 16 * blk_I(pw, s) + (lane & 15), j0 = 16 * blk_J(pw, s) + 4 * (lane >> 4);
                o.g[s] = (i * kQ + j0) * 4;
            }
            o.dt = lane * bk.H * 4;
        }
        const int ptid = pw * 64 + lane;
        constexpr int kRows = kQ + K - 1;
        FetchS fs;  // dt / ids of the chunk whose scalars come next
        FetchG fg;  // G pieces of the chunk whose M blocks come next
        int32_t seq_row = 0, seq_hi = 0;
        auto scal = [&](int s) { return sm + kOffSc + s * kScBytes; };
        const int64_t last = nCl - 1;
        constexpr int kRegLoads = reg_loads<HAS_SEQ, PASS>();
        static_assert(kRegLoads < 16, "vmcnt field");
        // In the state-only pass the producers have time to spare and the conv waves set the
        // pace: there the producers convolve the second half of each chunk (tokens 32 .. 63)
        // for channel 16 pw + li, into the X slot lane that consumer wave pw reads, and its
        // flag mask into the upper half of that lane's flag word.
        constexpr bool kProdConv = PASS == 1;
        const int p_pc = 16 * pw + (lane & 15), j0_pc = 32 + 8 * (lane >> 4);
        const int xoff_pc = (pw * 64 + lane) * 32 + 16;
        double pcw[K], pcb = 0.0;
        if (kProdConv) conv_weights<K, MODE>(a, h, p_pc, pcw, pcb);
        auto prod_conv_finish = [&](const uint8_t* raw, uint8_t* xs, uint8_t* fl, uint32_t near, bf16x8 x,
                                    bool clean) {
            lds_st(xs, xoff_pc, x);
            if (HAS_SEQ && MODE != 0 && !clean) {
                conv_masked_run<K, MODE>(raw, sm + kOffW, p_pc, j0_pc, xs, xoff_pc);
                near = 0;
            }
            lds_st(fl, (pw * 64 + lane) * 4 + 2, static_cast<uint16_t>(near));
        };
        // prologue: the block's first chunk's tiles, dt and raw rows and the second chunk's
        // raw rows; then the scalars of the first two chunks and the first chunk's M blocks.
        // Local chunk c is global chunk c0 + c (LDS slots go by the local index, memory by the
        // global one).
        fetch_tiles<PASS>(bk, o, c0, pw, sm_cb);
        fetch_s<HAS_SEQ>(bk, o, c0, lane, fs);
        fetch_raw<K, HAS_SEQ>(bk, o, c0 + 1, nCl > 1, pw, lane, sm_raw1, &seq_row, &seq_hi);
        stage_raw_first<K, MODE != 0, HAS_SEQ>(a, bk, b, h, static_cast<int>(c0 * kQ), pw, lane, sm_raw0);
        if (PASS == 0) {
            // the M blocks above the diagonal, (0, 1) and (2, 3): zero in both stages, hi and lo
            const int zb = (ptid >> 5) & 1, zrow = (zb ? 32 : 0) + ((ptid >> 1) & 15);
            const int zq = (zb ? 6 : 2) + (ptid & 1);
            lds_st(sm_m + (ptid >> 7) * kStageBytes + (((ptid >> 6) & 1) ? kStMlo : kStMhi), sw_m(zrow, zq),
                   u32x4{0u, 0u, 0u, 0u});
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (HAS_SEQ && nCl > 1) {
            if (ptid < kRows) reinterpret_cast<int32_t*>(sm_raw1 + kRwSeq)[ptid] = seq_row;
            if (pw == 0) {
                const uint32_t m = clean_runs<K>(seq_row, seq_hi, lane);
                if (lane == 0) *reinterpret_cast<uint32_t*>(sm_raw1 + kRwClean) = m;
            }
        }
        __syncthreads();  // raw rows of chunk 0 staged
        chunk_scalars<HAS_SEQ, PASS>(fs, c0, bk.L, Ah2, lane, scal(0));
        fetch_s<HAS_SEQ>(bk, o, c0 + min<int64_t>(1, last), lane, fs);
        fetch_g<PASS>(bk, o, c0, fg);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        chunk_scalars<HAS_SEQ, PASS>(fs, c0 + min<int64_t>(1, last), bk.L, Ah2, lane, scal(1));
        fetch_s<HAS_SEQ>(bk, o, c0 + min<int64_t>(2, last), lane, fs);
        __syncthreads();  // scalars of chunks 0 and 1 written
        if (PASS == 0) {
            MBlk mb;
            m_blocks<HAS_SEQ>(fg, pw, lane, scal(0), mb);
            store_m(mb, pw, lane, sm_m);
        }
        fetch_g<PASS>(bk, o, c0 + min<int64_t>(1, last), fg);
        if (kProdConv) {
            uint32_t near = 0;
            const bool clean = !(HAS_SEQ && MODE != 0) || ((lds_ld<uint32_t>(sm_raw0, kRwClean) >> (j0_pc / 8)) & 1u);
            const bf16x8 x = conv_fast<K, MODE, false>(sm_raw0, p_pc, j0_pc, pcw, pcb, &near);
            prod_conv_finish(sm_raw0, sm + kOffX, sm + kOffFl, near, x, clean);
        }
        __syncthreads();
        // chunk c: load chunk c+1's tiles (into stage (c+1)&1, free since chunk c-1 was
        // contracted) and chunk c+2's raw rows (into raw slot (c+2)%3, free since chunk c-1's
        // flagged outputs were redone), (state-only pass) convolve the second half of chunk
        // c+1, compute chunk c+2's scalars into scalar stage (c+2)%3 and chunk c+1's M blocks
        // from the scalars written in the previous iteration, so the two are independent
        // work; then, once this chunk's transfers have landed, load chunk c+2's G pieces and
        // chunk c+3's dt, which are used one iteration later.  Unrolled by three so the raw
        // slots and scalar stages are compile-time arrays.  The body has no branches between
        // the loads and the LDS work (the compiler then keeps track of which LDS array an
        // outstanding transfer writes): past the last chunk the indices are clamped, so the
        // loads repeat the last chunk into slots nobody reads and the conv writes an X slot
        // nobody reads.
        for (int64_t cn = 0; cn < nCl; cn += 3) {
#pragma unroll
            for (int third = 0; third < 3; ++third) {
                const int64_t c = cn + third;
                if (c >= nCl) break;
                const int64_t k = c + 1;
                const int64_t kt = k < nCl ? k : last;             // tiles of chunk c+1
                const int64_t kr = k + 1 < nCl ? k + 1 : last;     // raw rows, scalars of c+2
                uint8_t* stk = sm_m + (k & 1) * kStageBytes;
                uint8_t* raw_ld = third == 0 ? sm_raw2 : third == 1 ? sm_raw0 : sm_raw1;  // slot (c+2)%3
                fetch_tiles<PASS>(bk, o, c0 + kt, pw, sm_cb + (k & 1) * kCbBytes);
                fetch_raw<K, HAS_SEQ>(bk, o, c0 + kr, kr >= 1, pw, lane, raw_ld, &seq_row, &seq_hi);
                asm volatile("" ::: "memory");
                // (state-only pass) the unbranched part of the conv of chunk k's second half
                // before the wait, the rest after it
                const uint8_t* raw_cv = third == 0 ? sm_raw1 : third == 1 ? sm_raw2 : sm_raw0;  // slot k%3
                uint32_t near = 0;
                bf16x8 xpc{};
                bool pclean = true;
                if (kProdConv) {
                    pclean = !(HAS_SEQ && MODE != 0) || ((lds_ld<uint32_t>(raw_cv, kRwClean) >> (j0_pc / 8)) & 1u);
                    xpc = conv_fast<K, MODE, false>(raw_cv, p_pc, j0_pc, pcw, pcb, &near);
                }
                chunk_scalars<HAS_SEQ, PASS>(fs, c0 + kr, bk.L, Ah2, lane, scal((third + 2) % 3));
                MBlk mb;
                if (PASS == 0) m_blocks<HAS_SEQ>(fg, pw, lane, scal((third + 1) % 3), mb);
                // the registers the next iteration uses load while this iteration's transfers
                // land; vector memory loads complete in issue order, so waiting until only
                // those loads are outstanding means the transfers are in LDS.  The M blocks
                // are stored after that wait: LDS stores issued while transfers into LDS are
                // outstanding make the compiler wait for all of them.
                fetch_g<PASS>(bk, o, c0 + kr, fg);
                fetch_s<HAS_SEQ>(bk, o, c0 + (k + 2 < nCl ? k + 2 : last), lane, fs);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(kWaitVm0 | kRegLoads);
                if (PASS == 0) store_m(mb, pw, lane, stk);
                if (kProdConv)
                    prod_conv_finish(raw_cv, sm + kOffX + (k & 1) * kXBytes, sm + kOffFl + (k & 1) * kFlBytes, near, xpc,
                                     pclean);
                if (HAS_SEQ && k + 1 < nCl) {
                    if (ptid < kRows) reinterpret_cast<int32_t*>(raw_ld + kRwSeq)[ptid] = seq_row;
                    if (pw == 0) {
                        const uint32_t m = clean_runs<K>(seq_row, seq_hi, lane);
                        if (lane == 0) *reinterpret_cast<uint32_t*>(raw_ld + kRwClean) = m;
                    }
                }
                __syncthreads();
            }
        }
    } else {
        // conv wave cv: channel p = 16 cv + li over tokens 32 r + 8 g4 .. +7 of a chunk (runs
        // r = 0, 1), into the X slot lane that consumer wave cv reads.  (Eight conv waves, one
        // run each, were measured slower: at 16 waves per group the 128-VGPR budget spills.)
        const int cv = wave - 8;
        constexpr int kRuns = PASS == 1 ? 1 : 2;  // the producers take run 1 in the state-only pass
        const int p_conv = 16 * cv + li;
        const int j0_conv = 8 * g4;
        const int xoff = (cv * 64 + lane) * 32;
        double cw[K], cbias;
        conv_weights<K, MODE>(a, h, p_conv, cw, cbias);
        if (MODE != 0 && g4 == 0) {
#pragma unroll
            for (int k = 0; k < K; ++k) lds_st(sm + kOffW, p_conv * kWStride + 8 * k, cw[k]);
            lds_st(sm + kOffW, p_conv * kWStride + 8 * K, cbias);
        }
        // the flagged outputs go to the consumer lane that reads them (conv_fixups there), so
        // the rare double-precision recomputations stay off this role, which sets the pace
        auto conv_chunk = [&](const uint8_t* raw, uint8_t* xs, uint8_t* fl) {
            // both runs' fast paths (independent chains, no sequence masks); with seq_idx, a
            // run whose taps straddle a sequence boundary is redone with the masks (exactly
            // rounded, so its flags are cleared)
            // which runs' taps carry one sequence id (a word the producers computed)
            bool clean[kRuns];
            const uint32_t cm = (HAS_SEQ && MODE != 0) ? lds_ld<uint32_t>(raw, kRwClean) : 0xFFu;
#pragma unroll
            for (int r = 0; r < kRuns; ++r) clean[r] = (cm >> ((j0_conv + 32 * r) / 8)) & 1u;
            uint32_t nr[kRuns];
            bf16x8 xr[kRuns];
#pragma unroll
            for (int r = 0; r < kRuns; ++r) {
                nr[r] = 0;
                xr[r] = conv_fast<K, MODE, false>(raw, p_conv, j0_conv + 32 * r, cw, cbias, &nr[r]);
            }
#pragma unroll
            for (int r = 0; r < kRuns; ++r) lds_st(xs, xoff + 16 * r, xr[r]);
            if (HAS_SEQ && MODE != 0) {
#pragma unroll
                for (int r = 0; r < kRuns; ++r)
                    if (!clean[r]) {
                        conv_masked_run<K, MODE>(raw, sm + kOffW, p_conv, j0_conv + 32 * r, xs, xoff + 16 * r);
                        nr[r] = 0;
                    }
            }
            if (kRuns == 2)
                lds_st(fl, (cv * 64 + lane) * 4, nr[0] | (nr[kRuns - 1] << 16));
            else
                lds_st(fl, (cv * 64 + lane) * 4, static_cast<uint16_t>(nr[0]));
        };
        __syncthreads();  // raw rows of chunk 0 staged
        conv_chunk(sm_raw0, sm + kOffX, sm + kOffFl);
        __syncthreads();  // scalars of chunks 0 and 1 written
        __syncthreads();
        int slot = 1;  // raw slot of chunk cn + 1
        for (int64_t cn = 0; cn < nCl; ++cn) {
            if (cn + 1 < nCl)
                conv_chunk(slot == 0 ? sm_raw0 : slot == 1 ? sm_raw1 : sm_raw2,
                           sm + kOffX + ((cn + 1) & 1) * kXBytes, sm + kOffFl + ((cn + 1) & 1) * kFlBytes);
            slot = slot == 2 ? 0 : slot + 1;
            __syncthreads();
        }
    }

    // ---- final conv state F = u[L .. L+K-2] for this head's x channels and for slice h of
    // the B / C channels: all reads first, then a barrier, then the writes, so an in-place
    // state pair is never read after being overwritten.  Each block takes whole channel rows
    // (all K-1 entries of a channel): when L < K-1, F reads the initial state of the same
    // channel, which then no other block writes. ----
    if (MODE != 0 && a.conv_final && PASS == 0 && seg == 0) {
        constexpr int km1 = K - 1;
        const int64_t nx = kP * km1;
        const int64_t nbc_ch = 2 * a.G * kN;
        const int64_t per_ch = (nbc_ch + a.H - 1) / a.H;
        const int64_t bc_lo = min(h * per_ch, nbc_ch) * km1, bc_hi = min((h + 1) * per_ch, nbc_ch) * km1;
        const int64_t total = nx + (bc_hi - bc_lo);
        constexpr int kMaxItems = 6;  // >= ceil((64*7 + 2*128*7) / 768) for every G <= H
        uint16_t fv[kMaxItems];
        int64_t fidx[kMaxItems];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < kMaxItems; ++q) {
            const int64_t idx = tid + static_cast<int64_t>(q) * kMainThreads;
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

template <int K, int MODE, int PASS>
hipError_t launch_main(const ChunkedArgs& a, hipStream_t stream, int64_t nsl) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * nsl));
    if (a.seq_idx) ssd_main_kernel<K, MODE, true, PASS><<<grid, kMainThreads, 0, stream>>>(a);
    else ssd_main_kernel<K, MODE, false, PASS><<<grid, kMainThreads, 0, stream>>>(a);
    return hipGetLastError();
}

template <int K, int MODE>
hipError_t launch_passes(const ChunkedArgs& a, hipStream_t stream) {
    if (a.nseg > 1) {
        hipError_t e = launch_main<K, MODE, 1>(a, stream, a.nseg - 1);
        if (e != hipSuccess) return e;
    }
    return launch_main<K, MODE, 0>(a, stream, a.nseg);
}

template <int K>
hipError_t launch_k(const ChunkedArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    const int64_t nC = (a.L + kQ - 1) / kQ;
    ssd_prep_kernel<K><<<dim3(static_cast<unsigned>(nC), static_cast<unsigned>(a.G),
                              static_cast<unsigned>(a.B)),
                         kPrepThreads, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0) (void)hipEventRecord(ev0, stream);
    if (!a.fused_conv) {
        if constexpr (K == 2) e = launch_passes<K, 0>(a, stream);  // no conv: one halo row
        else e = hipErrorInvalidValue;
    }
    else if (a.act == SSM_ACT_SILU) e = launch_passes<K, 2>(a, stream);
    else e = launch_passes<K, 1>(a, stream);
    if (ev1) (void)hipEventRecord(ev1, stream);
    return e;
}

// Rows with few heads leave most CUs idle on the per-(row, head) sequential scan; they are
// split into segments (at least kMinSegChunks chunks each) so about kTargetBlocks blocks run.
constexpr int64_t kTargetBlocks = 256;
constexpr int64_t kMinSegChunks = 4;

int64_t chunked_nseg(int64_t B, int64_t L, int64_t H) {
    const int64_t nC = (L + kQ - 1) / kQ;
    int64_t nseg = kTargetBlocks / (B * H);
    nseg = nseg < nC / kMinSegChunks ? nseg : nC / kMinSegChunks;
    if (nseg < 2) return 1;
    const int64_t sc = (nC + nseg - 1) / nseg;
    return (nC + sc - 1) / sc;  // every segment non-empty
}

size_t tile_workspace_bytes(int64_t B, int64_t L, int64_t G) {
    const int64_t nC = (L + kQ - 1) / kQ;
    const int64_t units = B * nC * G;
    return static_cast<size_t>(units * (kWsC * 2 + kWsBt * 2 + kWsG * 4));
}

}  // namespace

bool chunked_supported(int64_t P, int64_t N, ssm_dtype_t dtype) {
    return dtype == SSM_BF16 && P == kP && N == kN;
}

size_t chunked_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t G, int64_t N) {
    if (N != kN) return 0;
    size_t bytes = (tile_workspace_bytes(B, L, G) + 255) / 256 * 256;
    const int64_t nseg = chunked_nseg(B, L, H);
    if (nseg > 1) bytes += static_cast<size_t>(B * H * nseg * (kP * kN + 1)) * 4;
    return bytes;
}

hipError_t launch_chunked(const ChunkedArgs& args, hipStream_t stream, hipEvent_t ev_before_main,
                          hipEvent_t ev_after_main) {
    if (args.B == 0 || args.L == 0) return hipSuccess;
    ChunkedArgs a = args;
    const int64_t nC = (a.L + kQ - 1) / kQ;
    a.nseg = chunked_nseg(a.B, a.L, a.H);
    a.seg_chunks = (nC + a.nseg - 1) / a.nseg;
    a.seg_state = nullptr;
    a.seg_decay = nullptr;
    if (a.nseg > 1) {
        const size_t off = (tile_workspace_bytes(a.B, a.L, a.G) + 255) / 256 * 256;
        a.seg_state = reinterpret_cast<float*>(static_cast<uint8_t*>(a.workspace) + off);
        a.seg_decay = a.seg_state + a.B * a.H * a.nseg * kP * kN;
    }
    switch (a.K) {
        case 2: return launch_k<2>(a, stream, ev_before_main, ev_after_main);
        case 3: return launch_k<3>(a, stream, ev_before_main, ev_after_main);
        case 4: return launch_k<4>(a, stream, ev_before_main, ev_after_main);
        case 5: return launch_k<5>(a, stream, ev_before_main, ev_after_main);
        case 6: return launch_k<6>(a, stream, ev_before_main, ev_after_main);
        case 7: return launch_k<7>(a, stream, ev_before_main, ev_after_main);
        case 8: return launch_k<8>(a, stream, ev_before_main, ev_after_main);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
