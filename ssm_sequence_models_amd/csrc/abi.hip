// abi.hip -- the C ABI (include/ssm_mi355x.h): argument checks, path selection, launches.
// Host code only; every computation runs in the kernels of conv.hip, recurrent.hip and
// ssd.hip.  Nothing here allocates device memory, synchronises, throws or prints.
#include <cmath>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_err;

ssm_status_t fail(ssm_status_t s, const std::string& msg) {
    g_err = msg;
    return s;
}
ssm_status_t ok() {
    g_err.clear();
    return SSM_OK;
}
ssm_status_t hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    g_err = std::string(where) + ": " + hipGetErrorString(e);
    return SSM_ERR_HIP;
}
size_t esize(ssm_dtype_t d) { return d == SSM_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_dtype(int d) { return d == SSM_F32 || d == SSM_BF16; }
bool valid_act(int a) { return a == SSM_ACT_NONE || a == SSM_ACT_SILU; }

// ---- optional kernel timing (measurement only) ----
std::mutex g_tmu;
bool g_timing = false;
struct EventPair {
    hipEvent_t e0, e1;
    int dev;
};
std::vector<EventPair> g_events;  // recorded, not yet read
std::vector<EventPair> g_spare;   // read, kept for reuse (created once, never per launch)

// Pointer arguments: name, pointer, required?, element alignment.
struct PtrCheck {
    const char* name;
    const void* p;
    bool required;
    size_t align;
};
ssm_status_t check_ptrs(const char* fn, std::initializer_list<PtrCheck> list) {
    for (const auto& c : list) {
        if (c.p == nullptr) {
            if (c.required) return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": " + c.name + " is NULL");
            continue;
        }
        if (!aligned(c.p, c.align))
            return fail(SSM_ERR_ALIGNMENT, std::string(fn) + ": " + c.name + " is not aligned to " +
                                               std::to_string(c.align) + " bytes");
    }
    return SSM_OK;
}

ssm_status_t check_scan_dims(const char* fn, int64_t batch, int64_t seqlen, int64_t nheads,
                             int64_t headdim, int64_t ngroups, int64_t dstate, int dtype) {
    if (!valid_dtype(dtype)) return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": bad dtype");
    if (batch < 0 || seqlen < 0)
        return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": negative batch or seqlen");
    if (nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1)
        return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": nheads, headdim, ngroups, dstate must be >= 1");
    if (nheads % ngroups != 0)
        return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": nheads is not a multiple of ngroups");
    return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int32_t s) {
    switch (s) {
        case SSM_OK: return "ok";
        case SSM_ERR_INVALID_ARG: return "invalid argument";
        case SSM_ERR_UNSUPPORTED: return "unsupported sizes or dtype";
        case SSM_ERR_ALIGNMENT: return "misaligned pointer";
        case SSM_ERR_WORKSPACE: return "workspace missing or too small";
        case SSM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* ssm_last_error(void) { return g_err.c_str(); }

ssm_status_t ssm_conv1d_fwd(const void* x, const float* w, const float* bias,
                            const void* initial_state, void* final_state,
                            const int32_t* seq_idx, void* out, int64_t batch, int64_t seqlen,
                            int64_t channels, int64_t width, ssm_dtype_t dtype, ssm_act_t act,
                            ssm_stream_t stream) {
    const char* fn = "ssm_conv1d_fwd";
    if (!valid_dtype(dtype)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_fwd: bad dtype");
    if (!valid_act(act)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_fwd: bad activation");
    if (batch < 0 || seqlen < 0 || channels < 1)
        return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_fwd: need batch >= 0, seqlen >= 0, channels >= 1");
    if (width < 2 || width > 8)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_conv1d_fwd: width must be in [2, 8]");
    const size_t es = esize(dtype);
    const bool work = batch > 0 && seqlen > 0;
    ssm_status_t st = check_ptrs(fn, {{"x", x, work, es},
                                      {"w", w, work, 4},
                                      {"bias", bias, false, 4},
                                      {"initial_state", initial_state, false, es},
                                      {"final_state", final_state, false, es},
                                      {"seq_idx", seq_idx, false, 4},
                                      {"out", out, work, es}});
    if (st != SSM_OK) return st;
    if (batch == 0) return ok();
    return hip_status(ssm::launch_conv1d_fwd(x, w, bias, initial_state, final_state, seq_idx, out,
                                             batch, seqlen, channels, width, dtype, act,
                                             reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

ssm_status_t ssm_conv1d_update(const void* x, void* conv_state, const float* w,
                               const float* bias, const int32_t* conv_state_indices,
                               const int32_t* cache_seqlens, void* out, int64_t batch,
                               int64_t channels, int64_t n_new, int64_t width,
                               int64_t state_len, int64_t n_slots, ssm_dtype_t dtype,
                               ssm_act_t act, ssm_stream_t stream) {
    const char* fn = "ssm_conv1d_update";
    if (!valid_dtype(dtype)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_update: bad dtype");
    if (!valid_act(act)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_update: bad activation");
    if (batch < 0 || n_new < 0 || channels < 1 || n_slots < 1)
        return fail(SSM_ERR_INVALID_ARG,
                    "ssm_conv1d_update: need batch >= 0, n_new >= 0, channels >= 1, n_slots >= 1");
    if (width < 2 || width > 8)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_conv1d_update: width must be in [2, 8]");
    if (state_len < width - 1)
        return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_update: state_len < width - 1");
    const size_t es = esize(dtype);
    const bool work = batch > 0 && n_new > 0;
    ssm_status_t st = check_ptrs(fn, {{"x", x, work, es},
                                      {"conv_state", conv_state, work, es},
                                      {"w", w, work, 4},
                                      {"bias", bias, false, 4},
                                      {"conv_state_indices", conv_state_indices, false, 4},
                                      {"cache_seqlens", cache_seqlens, false, 4},
                                      {"out", out, work, es}});
    if (st != SSM_OK) return st;
    if (!work) return ok();
    return hip_status(ssm::launch_conv1d_update(x, conv_state, w, bias, conv_state_indices,
                                                cache_seqlens, out, batch, channels, n_new, width,
                                                state_len, n_slots, dtype, act,
                                                reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

size_t ssm_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate, ssm_dtype_t dtype) {
    if (batch <= 0 || seqlen <= 0 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1 ||
        !valid_dtype(dtype))
        return 0;
    if (ssm::chunked_supported(headdim, dstate, dtype))
        return ssm::chunked_workspace_bytes(batch, seqlen, nheads, ngroups, dstate);
    // general-shape path of the fused call: the conv output is staged in the workspace
    return static_cast<size_t>(batch * seqlen * (nheads * headdim + 2 * ngroups * dstate)) *
           esize(dtype);
}

namespace {

// Shared tail of ssm_scan_fwd / ssm_conv_scan_fwd on the token-sequential path.
ssm_status_t run_recurrent_scan(const char* fn, const void* x, int64_t x_row, const void* Bm,
                                const void* Cm, int64_t bc_row, const float* dt, const float* A,
                                const float* initial_state, float* final_state,
                                const int32_t* seq_idx, void* y, int64_t batch, int64_t seqlen,
                                int64_t nheads, int64_t headdim, int64_t ngroups,
                                int64_t dstate, ssm_dtype_t dtype, hipStream_t s) {
    ssm::RecurrentArgs r{};
    r.x = x;
    r.x_sb = seqlen * x_row;
    r.x_st = x_row;
    r.x_sc = 1;
    r.dt = dt;
    r.A = A;
    r.Bm = Bm;
    r.B_sb = seqlen * bc_row;
    r.B_st = bc_row;
    r.B_sc = 1;
    r.Cm = Cm;
    r.C_sb = seqlen * bc_row;
    r.C_st = bc_row;
    r.C_sc = 1;
    r.state_in = initial_state;
    r.state_out = final_state;
    r.indices = nullptr;
    r.n_slots = batch;
    r.seq_idx = seq_idx;
    r.y = y;
    r.B = batch;
    r.T = seqlen;
    r.H = nheads;
    r.P = headdim;
    r.G = ngroups;
    r.N = dstate;
    return hip_status(ssm::launch_recurrent(r, dtype, s), fn);
}

hipEvent_t g_none = nullptr;

// Events for the timing record (both NULL when timing is off): a pair from the spare list
// of the current device when there is one, else a new pair (created once; ssm_timing_read
// returns pairs to the spare list instead of destroying them).
ssm_status_t timing_events(hipEvent_t* ev0, hipEvent_t* ev1) {
    *ev0 = *ev1 = g_none;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_timing) return SSM_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "timing");
    for (size_t i = g_spare.size(); i-- > 0;) {
        if (g_spare[i].dev == dev) {
            g_events.push_back(g_spare[i]);
            g_spare.erase(g_spare.begin() + static_cast<std::ptrdiff_t>(i));
            *ev0 = g_events.back().e0;
            *ev1 = g_events.back().e1;
            return SSM_OK;
        }
    }
    e = hipEventCreate(ev0);
    if (e == hipSuccess) e = hipEventCreate(ev1);
    if (e != hipSuccess) return hip_status(e, "timing");
    g_events.push_back({*ev0, *ev1, dev});
    return SSM_OK;
}

}  // namespace

ssm_status_t ssm_scan_fwd(const void* x, const float* dt, const float* A, const void* Bm,
                          const void* Cm, const float* initial_state, float* final_state,
                          const int32_t* seq_idx, void* y, int64_t batch, int64_t seqlen,
                          int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                          ssm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          ssm_stream_t stream) {
    const char* fn = "ssm_scan_fwd";
    ssm_status_t st = check_scan_dims(fn, batch, seqlen, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    const size_t es = esize(dtype);
    const bool work = batch > 0 && seqlen > 0;
    st = check_ptrs(fn, {{"x", x, work, es},
                         {"dt", dt, work, 4},
                         {"A", A, work, 4},
                         {"Bm", Bm, work, es},
                         {"Cm", Cm, work, es},
                         {"initial_state", initial_state, false, 16},
                         {"final_state", final_state, false, 16},
                         {"seq_idx", seq_idx, false, 4},
                         {"y", y, work, es}});
    if (st != SSM_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (batch == 0) return ok();
    if (seqlen == 0)
        return hip_status(ssm::launch_copy_or_zero_f32(final_state, initial_state,
                                                       batch * nheads * headdim * dstate, s),
                          fn);
    // the matrix-core path loads x, Bm and Cm rows in 16-byte pieces and stores y in 8-byte
    // pieces; other alignments take the token-sequential path
    if (ssm::chunked_supported(headdim, dstate, dtype) && aligned(x, 16) && aligned(Bm, 16) &&
        aligned(Cm, 16) && aligned(y, 8)) {
        const size_t need = ssm::chunked_workspace_bytes(batch, seqlen, nheads, ngroups, dstate);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
            return fail(SSM_ERR_WORKSPACE, "ssm_scan_fwd: workspace must be >= " +
                                               std::to_string(need) + " bytes, 16-byte aligned");
        ssm::ChunkedArgs a{};
        a.x = static_cast<const uint16_t*>(x);
        a.x_row = nheads * headdim;
        a.x_col0 = 0;
        a.bsrc = static_cast<const uint16_t*>(Bm);
        a.b_row = ngroups * dstate;
        a.b_col0 = 0;
        a.csrc = static_cast<const uint16_t*>(Cm);
        a.c_row = ngroups * dstate;
        a.c_col0 = 0;
        a.fused_conv = false;
        a.K = 2;  // no conv: one halo row staged and ignored
        a.C_conv = 0;
        a.act = SSM_ACT_NONE;
        a.dt = dt;
        a.A = A;
        a.init_state = initial_state;
        a.final_state = final_state;
        a.seq_idx = seq_idx;
        a.y = static_cast<uint16_t*>(y);
        a.B = batch;
        a.L = seqlen;
        a.H = nheads;
        a.P = headdim;
        a.G = ngroups;
        a.N = dstate;
        a.workspace = workspace;
        hipEvent_t e0, e1;
        st = timing_events(&e0, &e1);
        if (st != SSM_OK) return st;
        return hip_status(ssm::launch_chunked(a, s, e0, e1), fn);
    }
    if (!ssm::recurrent_supported(headdim, dstate))
        return fail(SSM_ERR_UNSUPPORTED, "ssm_scan_fwd: dstate must be 4 * 2^k <= 256 and headdim*dstate <= 16384");
    return run_recurrent_scan(fn, x, nheads * headdim, Bm, Cm, ngroups * dstate, dt, A,
                              initial_state, final_state, seq_idx, y, batch, seqlen, nheads,
                              headdim, ngroups, dstate, dtype, s);
}

namespace {

// Body of ssm_conv_scan_fwd and ssm_conv_scan_fwd_noalloc; `timed` lets the main-kernel
// timing record (when switched on) create its events.
ssm_status_t conv_scan_fwd_impl(const char* fn, const void* xBC, const float* conv_w,
                                const float* conv_bias, const void* conv_initial_state,
                                void* conv_final_state, const float* dt, const float* A,
                                const float* initial_state, float* final_state,
                                const int32_t* seq_idx, void* y, int64_t batch, int64_t seqlen,
                                int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                                int64_t width, ssm_dtype_t dtype, ssm_act_t act, void* workspace,
                                size_t workspace_bytes, bool timed, ssm_stream_t stream,
                                const int32_t* state_slots = nullptr, int64_t n_state_slots = 0) {
    // n_state_slots > 0 (the pooled prefill, chunked shapes only): the SSM states are rows
    // state_slots[b] of an [n_state_slots, H, P, N] pool, read and written in place
    ssm_status_t st = check_scan_dims(fn, batch, seqlen, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    if (!valid_act(act)) return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": bad activation");
    if (width < 2 || width > 8)
        return fail(SSM_ERR_UNSUPPORTED, std::string(fn) + ": width must be in [2, 8]");
    const size_t es = esize(dtype);
    const bool work = batch > 0 && seqlen > 0;
    st = check_ptrs(fn, {{"xBC", xBC, work, es},
                         {"conv_w", conv_w, work, 4},
                         {"conv_bias", conv_bias, false, 4},
                         {"conv_initial_state", conv_initial_state, false, es},
                         {"conv_final_state", conv_final_state, false, es},
                         {"dt", dt, work, 4},
                         {"A", A, work, 4},
                         {"initial_state", initial_state, false, 16},
                         {"final_state", final_state, false, 16},
                         {"seq_idx", seq_idx, false, 4},
                         {"y", y, work, es}});
    if (st != SSM_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t C_conv = nheads * headdim + 2 * ngroups * dstate;
    if (batch == 0) return ok();
    if (seqlen == 0) {
        hipError_t e = ssm::launch_conv1d_fwd(nullptr, conv_w, conv_bias, conv_initial_state,
                                              conv_final_state, nullptr, nullptr, batch, 0,
                                              C_conv, width, dtype, act, s);
        // pool rows stay where they are: nothing to copy
        if (e == hipSuccess && n_state_slots <= 0)
            e = ssm::launch_copy_or_zero_f32(final_state, initial_state,
                                             batch * nheads * headdim * dstate, s);
        return hip_status(e, fn);
    }
    if (ssm::chunked_supported(headdim, dstate, dtype)) {
        const size_t need = ssm::chunked_workspace_bytes(batch, seqlen, nheads, ngroups, dstate);
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
            return fail(SSM_ERR_WORKSPACE, std::string(fn) + ": workspace must be >= " +
                                               std::to_string(need) + " bytes, 16-byte aligned");
        if (!aligned(xBC, 16) || C_conv % 8 != 0 || !aligned(y, 8))
            return fail(SSM_ERR_ALIGNMENT,
                        std::string(fn) + ": xBC must be 16-byte aligned with a channel count "
                        "divisible by 8, y 8-byte aligned");
        ssm::ChunkedArgs a{};
        a.x = static_cast<const uint16_t*>(xBC);
        a.x_row = C_conv;
        a.x_col0 = 0;
        a.bsrc = a.x;
        a.b_row = C_conv;
        a.b_col0 = nheads * headdim;
        a.csrc = a.x;
        a.c_row = C_conv;
        a.c_col0 = nheads * headdim + ngroups * dstate;
        a.fused_conv = true;
        a.conv_w = conv_w;
        a.conv_b = conv_bias;
        a.conv_init = static_cast<const uint16_t*>(conv_initial_state);
        a.conv_final = static_cast<uint16_t*>(conv_final_state);
        a.C_conv = C_conv;
        a.K = width;
        a.act = act;
        a.dt = dt;
        a.A = A;
        a.init_state = initial_state;
        a.final_state = final_state;
        a.state_slots = state_slots;
        a.n_state_slots = n_state_slots;
        a.seq_idx = seq_idx;
        a.y = static_cast<uint16_t*>(y);
        a.B = batch;
        a.L = seqlen;
        a.H = nheads;
        a.P = headdim;
        a.G = ngroups;
        a.N = dstate;
        a.workspace = workspace;
        hipEvent_t e0 = g_none, e1 = g_none;
        if (timed) {
            st = timing_events(&e0, &e1);
            if (st != SSM_OK) return st;
        }
        return hip_status(ssm::launch_chunked(a, s, e0, e1), fn);
    }
    // general shapes: conv into the workspace, then the token-sequential scan reading its
    // x | B | C channel ranges in place
    if (n_state_slots > 0)
        return fail(SSM_ERR_UNSUPPORTED, std::string(fn) + ": pool rows need the chunked path");
    if (!ssm::recurrent_supported(headdim, dstate))
        return fail(SSM_ERR_UNSUPPORTED, std::string(fn) + ": dstate must be 4 * 2^k <= 256 and headdim*dstate <= 16384");
    const size_t need = static_cast<size_t>(batch * seqlen * C_conv) * es;
    if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
        return fail(SSM_ERR_WORKSPACE, std::string(fn) + ": workspace must be >= " +
                                           std::to_string(need) + " bytes, 16-byte aligned");
    hipError_t e = ssm::launch_conv1d_fwd(xBC, conv_w, conv_bias, conv_initial_state,
                                          conv_final_state, seq_idx, workspace, batch, seqlen,
                                          C_conv, width, dtype, act, s);
    if (e != hipSuccess) return hip_status(e, fn);
    const uint8_t* base = static_cast<const uint8_t*>(workspace);
    return run_recurrent_scan(fn, base, C_conv, base + nheads * headdim * es,
                              base + (nheads * headdim + ngroups * dstate) * es, C_conv, dt, A,
                              initial_state, final_state, seq_idx, y, batch, seqlen, nheads,
                              headdim, ngroups, dstate, dtype, s);
}

}  // namespace

ssm_status_t ssm_conv_scan_fwd(const void* xBC, const float* conv_w, const float* conv_bias,
                               const void* conv_initial_state, void* conv_final_state,
                               const float* dt, const float* A, const float* initial_state,
                               float* final_state, const int32_t* seq_idx, void* y,
                               int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate, int64_t width,
                               ssm_dtype_t dtype, ssm_act_t act, void* workspace,
                               size_t workspace_bytes, ssm_stream_t stream) {
    return conv_scan_fwd_impl("ssm_conv_scan_fwd", xBC, conv_w, conv_bias, conv_initial_state,
                              conv_final_state, dt, A, initial_state, final_state, seq_idx, y,
                              batch, seqlen, nheads, headdim, ngroups, dstate, width, dtype, act,
                              workspace, workspace_bytes, true, stream);
}

// ---------------------------------------------------------------------------------------
// Allocation-free fused prefill: the workspace is a static device array of the library.
// ---------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, created when the library's code object is loaded on that GPU and held
// until the process ends.  Host code never passes `scratch` itself to a kernel (its host-side
// name is not a device address); it uses the per-device address from scratch_address().
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device.
ssm_status_t scratch_address(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SSM_ERR_UNSUPPORTED, std::string(fn) + ": device ordinal " +
                                             std::to_string(dev) + " beyond the scratch table");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        if (p == nullptr) return fail(SSM_ERR_HIP, std::string(fn) + ": scratch has no address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSM_OK;
}

}  // namespace

size_t ssm_noalloc_scratch_bytes(void) { return kScratchBytes; }

ssm_status_t ssm_conv_scan_fwd_noalloc(const void* xBC, const float* conv_w,
                                       const float* conv_bias, const void* conv_initial_state,
                                       void* conv_final_state, const float* dt, const float* A,
                                       const float* initial_state, float* final_state,
                                       const int32_t* seq_idx, void* y, int64_t batch,
                                       int64_t seqlen, int64_t nheads, int64_t headdim,
                                       int64_t ngroups, int64_t dstate, int64_t width,
                                       ssm_dtype_t dtype, ssm_act_t act, ssm_stream_t stream) {
    const char* fn = "ssm_conv_scan_fwd_noalloc";
    const size_t need = ssm_scan_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate,
                                                dtype);
    if (need > kScratchBytes)
        return fail(SSM_ERR_WORKSPACE, std::string(fn) + ": these sizes need " +
                                           std::to_string(need) + " bytes of scratch; the static "
                                           "scratch holds " + std::to_string(kScratchBytes) +
                                           " (ssm_conv_scan_fwd takes a workspace of any size)");
    void* ws = nullptr;
    if (batch > 0 && seqlen > 0) {
        // argument errors are reported before the scratch is looked up
        ssm_status_t st = check_scan_dims(fn, batch, seqlen, nheads, headdim, ngroups, dstate,
                                          dtype);
        if (st != SSM_OK) return st;
        st = scratch_address(fn, &ws);
        if (st != SSM_OK) return st;
    }
    return conv_scan_fwd_impl(fn, xBC, conv_w, conv_bias, conv_initial_state, conv_final_state,
                              dt, A, initial_state, final_state, seq_idx, y, batch, seqlen,
                              nheads, headdim, ngroups, dstate, width, dtype, act, ws,
                              ws ? kScratchBytes : 0, false, stream);
}

ssm_status_t ssm_step(const void* x, int64_t x_sb, int64_t x_st, int64_t x_sc, const float* dt,
                      const float* A, const void* Bm, int64_t B_sb, int64_t B_st, int64_t B_sc,
                      const void* Cm, int64_t C_sb, int64_t C_st, int64_t C_sc, float* state,
                      const int32_t* state_indices, void* y, int64_t batch, int64_t n_new,
                      int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                      int64_t n_slots, ssm_dtype_t dtype, ssm_stream_t stream) {
    const char* fn = "ssm_step";
    ssm_status_t st = check_scan_dims(fn, batch, n_new, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    if (n_slots < 1) return fail(SSM_ERR_INVALID_ARG, "ssm_step: n_slots must be >= 1");
    if (!ssm::recurrent_supported(headdim, dstate))
        return fail(SSM_ERR_UNSUPPORTED, "ssm_step: dstate must be 4 * 2^k <= 256 and headdim*dstate <= 16384");
    const size_t es = esize(dtype);
    const bool work = batch > 0 && n_new > 0;
    st = check_ptrs(fn, {{"x", x, work, es},
                         {"dt", dt, work, 4},
                         {"A", A, work, 4},
                         {"Bm", Bm, work, es},
                         {"Cm", Cm, work, es},
                         {"state", state, work, 16},
                         {"state_indices", state_indices, false, 4},
                         {"y", y, work, es}});
    if (st != SSM_OK) return st;
    if (!work) return ok();
    ssm::RecurrentArgs r{};
    r.x = x;
    r.x_sb = x_sb;
    r.x_st = x_st;
    r.x_sc = x_sc;
    r.dt = dt;
    r.A = A;
    r.Bm = Bm;
    r.B_sb = B_sb;
    r.B_st = B_st;
    r.B_sc = B_sc;
    r.Cm = Cm;
    r.C_sb = C_sb;
    r.C_st = C_st;
    r.C_sc = C_sc;
    r.state_in = state;
    r.state_out = state;
    r.indices = state_indices;
    r.n_slots = n_slots;
    r.seq_idx = nullptr;
    r.y = y;
    r.B = batch;
    r.T = n_new;
    r.H = nheads;
    r.P = headdim;
    r.G = ngroups;
    r.N = dstate;
    return hip_status(ssm::launch_recurrent(r, dtype, reinterpret_cast<hipStream_t>(stream)), fn);
}

ssm_status_t ssm_decode_step(const void* x_new, void* conv_state, const float* conv_w,
                             const float* conv_bias, const int32_t* conv_state_indices,
                             const int32_t* cache_seqlens, const float* dt, const float* A,
                             float* ssm_state, const int32_t* state_indices, void* conv_out,
                             void* y, int64_t batch, int64_t n_new, int64_t nheads,
                             int64_t headdim, int64_t ngroups, int64_t dstate, int64_t width,
                             int64_t state_len, int64_t n_conv_slots, int64_t n_ssm_slots,
                             ssm_dtype_t dtype, ssm_act_t act, ssm_stream_t stream) {
    const char* fn = "ssm_decode_step";
    ssm_status_t st = check_scan_dims(fn, batch, n_new, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    if (!valid_act(act)) return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": bad activation");
    if (n_conv_slots < 1 || n_ssm_slots < 1)
        return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": n_conv_slots and n_ssm_slots must be >= 1");
    if (width < 2 || width > 8)
        return fail(SSM_ERR_UNSUPPORTED, std::string(fn) + ": width must be in [2, 8]");
    if (state_len < width - 1)
        return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": state_len < width - 1");
    if (!ssm::recurrent_supported(headdim, dstate))
        return fail(SSM_ERR_UNSUPPORTED, std::string(fn) + ": dstate must be 4 * 2^k <= 256 and headdim*dstate <= 16384");
    const size_t es = esize(dtype);
    const bool work = batch > 0 && n_new > 0;
    st = check_ptrs(fn, {{"x_new", x_new, work, es},
                         {"conv_state", conv_state, work, es},
                         {"conv_w", conv_w, work, 4},
                         {"conv_bias", conv_bias, false, 4},
                         {"conv_state_indices", conv_state_indices, false, 4},
                         {"cache_seqlens", cache_seqlens, false, 4},
                         {"dt", dt, work, 4},
                         {"A", A, work, 4},
                         {"ssm_state", ssm_state, work, 16},
                         {"state_indices", state_indices, false, 4},
                         {"conv_out", conv_out, work, es},
                         {"y", y, work, es}});
    if (st != SSM_OK) return st;
    if (!work) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t C = nheads * headdim + 2 * ngroups * dstate;
    const int64_t HP = nheads * headdim, GN = ngroups * dstate;
    ssm::RecurrentArgs r{};
    r.x = conv_out;  // x | B | C channel ranges of the conv output [batch, C, n_new]
    r.x_sb = C * n_new;
    r.x_st = 1;
    r.x_sc = n_new;
    r.dt = dt;
    r.A = A;
    r.Bm = static_cast<const uint8_t*>(conv_out) + HP * n_new * es;
    r.B_sb = C * n_new;
    r.B_st = 1;
    r.B_sc = n_new;
    r.Cm = static_cast<const uint8_t*>(conv_out) + (HP + GN) * n_new * es;
    r.C_sb = C * n_new;
    r.C_st = 1;
    r.C_sc = n_new;
    r.state_in = ssm_state;
    r.state_out = ssm_state;
    r.indices = state_indices ? state_indices : conv_state_indices;
    r.n_slots = n_ssm_slots;
    r.seq_idx = nullptr;
    r.y = y;
    r.B = batch;
    r.T = n_new;
    r.H = nheads;
    r.P = headdim;
    r.G = ngroups;
    r.N = dstate;
    hipError_t e = ssm::launch_conv1d_update(x_new, conv_state, conv_w, conv_bias,
                                             conv_state_indices, cache_seqlens, conv_out, batch,
                                             C, n_new, width, state_len, n_conv_slots, dtype, act,
                                             s);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(ssm::launch_recurrent(r, dtype, s), fn);
}

ssm_status_t ssm_scan_fwd_vector_decay(const void* x, const float* dt, const float* log_decay,
                                       const float* A_vec, const void* Bm, const void* Cm,
                                       const float* initial_state, float* final_state,
                                       const int32_t* seq_idx, void* y, int64_t batch,
                                       int64_t seqlen, int64_t nheads, int64_t headdim,
                                       int64_t ngroups, int64_t dstate, ssm_dtype_t dtype,
                                       ssm_stream_t stream) {
    const char* fn = "ssm_scan_fwd_vector_decay";
    ssm_status_t st = check_scan_dims(fn, batch, seqlen, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    const size_t es = esize(dtype);
    const bool rows = batch > 0;
    const bool work = rows && seqlen > 0;
    // the decay source matters only when there are tokens (an empty tensor has no address)
    if (work && (log_decay == nullptr) == (A_vec == nullptr))
        return fail(SSM_ERR_INVALID_ARG, "ssm_scan_fwd_vector_decay: give exactly one of log_decay and A_vec");
    if (work && A_vec != nullptr && dt == nullptr)
        return fail(SSM_ERR_INVALID_ARG, "ssm_scan_fwd_vector_decay: the A_vec form needs dt");
    if (!ssm::recurrent_supported(headdim, dstate, true))
        return fail(SSM_ERR_UNSUPPORTED, "ssm_scan_fwd_vector_decay: dstate must be 4 * 2^k <= 256 and headdim*dstate <= 16384");
    st = check_ptrs(fn, {{"x", x, work, es},
                         {"dt", dt, false, 4},
                         {"log_decay", log_decay, false, 4},
                         {"A_vec", A_vec, false, 4},
                         {"B", Bm, work, es},
                         {"C", Cm, work, es},
                         {"initial_state", initial_state, false, 16},
                         {"final_state", final_state, false, 16},
                         {"seq_idx", seq_idx, false, 4},
                         {"y", y, work, es}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    if (!work)  // no tokens: the final state is the initial state (or zero)
        return hip_status(ssm::launch_copy_or_zero_f32(final_state, initial_state,
                                                       batch * nheads * headdim * dstate,
                                                       reinterpret_cast<hipStream_t>(stream)),
                          fn);
    ssm::RecurrentArgs r{};
    r.x = x;
    r.x_sb = seqlen * nheads * headdim;
    r.x_st = nheads * headdim;
    r.x_sc = 1;
    r.dt = dt;
    r.A = nullptr;
    r.Bm = Bm;
    r.B_sb = seqlen * ngroups * dstate;
    r.B_st = ngroups * dstate;
    r.B_sc = 1;
    r.Cm = Cm;
    r.C_sb = r.B_sb;
    r.C_st = r.B_st;
    r.C_sc = 1;
    r.state_in = initial_state;
    r.state_out = final_state;
    r.indices = nullptr;
    r.n_slots = batch;
    r.seq_idx = seq_idx;
    r.y = y;
    r.B = batch;
    r.T = seqlen;
    r.H = nheads;
    r.P = headdim;
    r.G = ngroups;
    r.N = dstate;
    r.log_decay = log_decay;
    r.A_vec = A_vec;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (ssm::vdecay_supported(headdim, dstate))
        return hip_status(ssm::launch_vdecay(r, dtype, s), fn);
    return hip_status(ssm::launch_recurrent(r, dtype, s), fn);
}

namespace {
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
}  // namespace

size_t ssm_conv_scan_fwd_pooled_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                               int64_t headdim, int64_t ngroups, int64_t dstate,
                                               int64_t width, ssm_dtype_t dtype) {
    if (batch <= 0 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1 || width < 2 ||
        width > 8 || !valid_dtype(dtype))
        return 0;
    const int64_t C_conv = nheads * headdim + 2 * ngroups * dstate;
    const size_t scan = round256(ssm_scan_workspace_size(batch, seqlen, nheads, headdim, ngroups,
                                                         dstate, dtype));
    const size_t hist = round256(static_cast<size_t>(batch * C_conv * (width - 1)) * esize(dtype));
    const size_t st = round256(static_cast<size_t>(batch * nheads * headdim * dstate) * 4);
    return scan + hist + st;
}

ssm_status_t ssm_conv_scan_fwd_pooled(const void* xBC, const float* conv_w,
                                      const float* conv_bias, const float* dt, const float* A,
                                      void* conv_state, float* ssm_state,
                                      const int32_t* state_indices, const int32_t* cache_seqlens,
                                      const int32_t* seq_idx, void* y, int64_t batch,
                                      int64_t seqlen, int64_t nheads, int64_t headdim,
                                      int64_t ngroups, int64_t dstate, int64_t width,
                                      int64_t state_len, int64_t n_slots, ssm_dtype_t dtype,
                                      ssm_act_t act, void* workspace, size_t workspace_bytes,
                                      ssm_stream_t stream) {
    const char* fn = "ssm_conv_scan_fwd_pooled";
    ssm_status_t st = check_scan_dims(fn, batch, seqlen, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    if (!valid_act(act)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv_scan_fwd_pooled: bad activation");
    if (width < 2 || width > 8)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_conv_scan_fwd_pooled: width must be in [2, 8]");
    if (n_slots < 1 || state_len < width - 1)
        return fail(SSM_ERR_INVALID_ARG,
                    "ssm_conv_scan_fwd_pooled: need n_slots >= 1 and state_len >= width - 1");
    const size_t es = esize(dtype);
    const bool rows = batch > 0;
    // every pointer is checked before the first launch, so a rejected call leaves the pools
    // and the workspace untouched
    st = check_ptrs(fn, {{"xBC", xBC, rows, es},
                         {"conv_w", conv_w, rows, 4},
                         {"conv_bias", conv_bias, false, 4},
                         {"dt", dt, rows, 4},
                         {"A", A, rows, 4},
                         {"conv_state", conv_state, rows, es},
                         {"ssm_state", ssm_state, rows, 4},
                         {"state_indices", state_indices, false, 4},
                         {"cache_seqlens", cache_seqlens, false, 4},
                         {"seq_idx", seq_idx, false, 4},
                         {"y", y, rows, es}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    const size_t need = ssm_conv_scan_fwd_pooled_workspace_size(batch, seqlen, nheads, headdim,
                                                                ngroups, dstate, width, dtype);
    if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
        return fail(SSM_ERR_WORKSPACE, std::string(fn) + ": workspace must be >= " +
                                           std::to_string(need) + " bytes, 256-byte aligned");
    const int64_t C_conv = nheads * headdim + 2 * ngroups * dstate;
    const int64_t per = nheads * headdim * dstate;
    const size_t scan = round256(ssm_scan_workspace_size(batch, seqlen, nheads, headdim, ngroups,
                                                         dstate, dtype));
    const size_t hist_b = round256(static_cast<size_t>(batch * C_conv * (width - 1)) * es);
    uint8_t* base = static_cast<uint8_t*>(workspace);
    void* hist = base + scan;
    float* sstate = reinterpret_cast<float*>(base + scan + hist_b);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // The chunked scan reads and writes the SSM pool rows itself (no gather or scatter of
    // states); other shapes run the states through the workspace.
    const bool in_pool = ssm::chunked_supported(headdim, dstate, dtype) && aligned(ssm_state, 16);
    const int64_t moved = in_pool ? 0 : per;
    hipError_t e = ssm::launch_pool_gather(conv_state, ssm_state, state_indices, cache_seqlens,
                                           hist, sstate, batch, C_conv, width, state_len, moved,
                                           n_slots, dtype, s);
    if (e != hipSuccess) return hip_status(e, fn);
    if (in_pool)
        st = conv_scan_fwd_impl(fn, xBC, conv_w, conv_bias, hist, nullptr, dt, A, ssm_state,
                                ssm_state, seq_idx, y, batch, seqlen, nheads, headdim, ngroups,
                                dstate, width, dtype, act, scan > 0 ? workspace : nullptr, scan,
                                true, stream, state_indices, n_slots);
    else
        st = ssm_conv_scan_fwd(xBC, conv_w, conv_bias, hist, nullptr, dt, A, sstate, sstate,
                               seq_idx, y, batch, seqlen, nheads, headdim, ngroups, dstate, width,
                               dtype, act, scan > 0 ? workspace : nullptr, scan, stream);
    if (st != SSM_OK) return st;
    return hip_status(ssm::launch_pool_scatter(conv_state, ssm_state, state_indices, cache_seqlens,
                                               xBC, sstate, batch, seqlen, C_conv, state_len,
                                               moved, n_slots, dtype, s),
                      fn);
}

size_t ssm_conv1d_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t channels,
                                     int64_t width) {
    if (batch <= 0 || seqlen <= 0 || channels < 1 || width < 2 || width > 8) return 0;
    return static_cast<size_t>(ssm::conv1d_bwd_workspace_bytes(batch, seqlen, channels, width));
}

ssm_status_t ssm_conv1d_bwd(const void* x, const float* w, const float* bias,
                            const void* initial_state, const int32_t* seq_idx, const void* dout,
                            const void* dfinal_state, void* dx, void* dinitial_state, float* dw,
                            float* dbias, void* workspace, size_t workspace_bytes, int64_t batch,
                            int64_t seqlen, int64_t channels, int64_t width, ssm_dtype_t dtype,
                            ssm_act_t act, ssm_stream_t stream) {
    const char* fn = "ssm_conv1d_bwd";
    if (!valid_dtype(dtype)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_bwd: bad dtype");
    if (!valid_act(act)) return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_bwd: bad activation");
    if (batch < 0 || seqlen < 0 || channels < 1)
        return fail(SSM_ERR_INVALID_ARG, "ssm_conv1d_bwd: need batch >= 0, seqlen >= 0, channels >= 1");
    if (width < 2 || width > 8)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_conv1d_bwd: width must be in [2, 8]");
    const size_t es = esize(dtype);
    const bool rows = batch > 0;
    const bool work = rows && seqlen > 0;
    ssm_status_t st = check_ptrs(fn, {{"x", x, work, es},
                                      {"w", w, work, 4},
                                      {"bias", bias, false, 4},
                                      {"initial_state", initial_state, false, es},
                                      {"seq_idx", seq_idx, false, 4},
                                      {"dout", dout, work, es},
                                      {"dfinal_state", dfinal_state, false, es},
                                      {"dx", dx, work, es},
                                      {"dinitial_state", dinitial_state, false, es},
                                      {"dw", dw, rows, 4},
                                      {"dbias", dbias, false, 4},
                                      {"workspace", workspace, false, 4}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    const size_t need = ssm_conv1d_bwd_workspace_size(batch, seqlen, channels, width);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, "ssm_conv1d_bwd: workspace missing or smaller than "
                                       "ssm_conv1d_bwd_workspace_size");
    return hip_status(ssm::launch_conv1d_bwd(x, w, bias, initial_state, seq_idx, dout, dfinal_state,
                                             dx, dinitial_state, dw, dbias, workspace, batch, seqlen,
                                             channels, width, dtype, act,
                                             reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

ssm_status_t ssm_scan_bwd_initial_state(const float* dt, const float* A, const void* C,
                                        const void* dy, const int32_t* seq_idx,
                                        const float* dfinal_state, float* dinitial_state,
                                        int64_t batch, int64_t seqlen, int64_t nheads,
                                        int64_t headdim, int64_t ngroups, int64_t dstate,
                                        ssm_dtype_t dtype, ssm_stream_t stream) {
    const char* fn = "ssm_scan_bwd_initial_state";
    ssm_status_t st = check_scan_dims(fn, batch, seqlen, nheads, headdim, ngroups, dstate, dtype);
    if (st != SSM_OK) return st;
    const size_t es = esize(dtype);
    const bool rows = batch > 0;
    const bool work = rows && seqlen > 0;
    st = check_ptrs(fn, {{"dt", dt, work, 4},
                         {"A", A, rows, 4},
                         {"C", C, work, es},
                         {"dy", dy, work, es},
                         {"seq_idx", seq_idx, false, 4},
                         {"dfinal_state", dfinal_state, false, 4},
                         {"dinitial_state", dinitial_state, rows, 4}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    return hip_status(ssm::launch_scan_bwd_h0(dt, A, C, seq_idx, dy, dfinal_state, dinitial_state,
                                              batch, seqlen, nheads, headdim, ngroups, dstate,
                                              dtype, reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

namespace {
ssm_status_t check_state_dims(const char* fn, int64_t batch, int64_t nheads, int64_t headdim,
                              int64_t dstate) {
    if (batch < 0) return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": negative batch");
    if (nheads < 1 || headdim < 1 || dstate < 1)
        return fail(SSM_ERR_INVALID_ARG, std::string(fn) + ": nheads, headdim, dstate must be >= 1");
    return SSM_OK;
}
}  // namespace

ssm_status_t ssm_state_stats_update(const float* final_state, int64_t batch, int64_t nheads,
                                    int64_t headdim, int64_t dstate, float beta, float* mean,
                                    float* var, ssm_stream_t stream) {
    const char* fn = "ssm_state_stats_update";
    ssm_status_t st = check_state_dims(fn, batch, nheads, headdim, dstate);
    if (st != SSM_OK) return st;
    if (!(beta == beta)) return fail(SSM_ERR_INVALID_ARG, "ssm_state_stats_update: beta is NaN");
    const bool rows = batch > 0;
    st = check_ptrs(fn, {{"final_state", final_state, rows, 4},
                         {"mean", mean, rows, 4},
                         {"var", var, rows, 4}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    if (nheads > 0x7FFFFFFF)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_state_stats_update: too many heads");
    return hip_status(ssm::launch_state_stats(final_state, batch, nheads, headdim * dstate,
                                              static_cast<double>(beta), mean, var,
                                              reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

ssm_status_t ssm_initial_state_noise(float* out, int64_t batch, int64_t nheads, int64_t headdim,
                                     int64_t dstate, const float* mean, const float* var,
                                     float sigma, uint64_t seed, uint64_t offset,
                                     ssm_stream_t stream) {
    const char* fn = "ssm_initial_state_noise";
    ssm_status_t st = check_state_dims(fn, batch, nheads, headdim, dstate);
    if (st != SSM_OK) return st;
    if ((mean == nullptr) != (var == nullptr))
        return fail(SSM_ERR_INVALID_ARG, "ssm_initial_state_noise: give both mean and var, or neither");
    const bool rows = batch > 0;
    st = check_ptrs(fn, {{"out", out, rows, 4}, {"mean", mean, false, 4}, {"var", var, false, 4}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    const int64_t n = batch * nheads * headdim * dstate;
    if ((n + 7) / 8 > static_cast<int64_t>(0xFFFFFFFFll) * 256)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_initial_state_noise: tensor too large");
    return hip_status(ssm::launch_state_noise(out, n, nheads, headdim * dstate, mean, var, sigma,
                                              seed, offset, reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

ssm_status_t ssm_state_reset(const void* src, void* dst, uint8_t* reset_mask, int64_t batch,
                             int64_t row_bytes, double p, uint64_t seed, uint64_t offset,
                             ssm_stream_t stream) {
    const char* fn = "ssm_state_reset";
    if (batch < 0 || row_bytes < 0 || (row_bytes & 1))
        return fail(SSM_ERR_INVALID_ARG, "ssm_state_reset: need batch >= 0 and an even row_bytes >= 0");
    if (!(p == p)) return fail(SSM_ERR_INVALID_ARG, "ssm_state_reset: p is NaN");
    const bool rows = batch > 0;
    ssm_status_t st = check_ptrs(fn, {{"src", src, rows && row_bytes > 0, 2},
                                      {"dst", dst, rows && row_bytes > 0, 2}});
    if (st != SSM_OK) return st;
    if (!rows) return ok();
    // threshold = floor(p 2^32), p clipped to [0, 1] (the scaling by 2^32 is exact)
    double t = std::floor((p < 0.0 ? 0.0 : p > 1.0 ? 1.0 : p) * 4294967296.0);
    const uint64_t threshold = static_cast<uint64_t>(t);
    const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
    const int unit = ((a & 15) == 0 && row_bytes % 16 == 0) ? 16
                     : ((a & 3) == 0 && row_bytes % 4 == 0) ? 4 : 2;
    if (ssm::state_reset_blocks(batch, row_bytes, unit) > 0x7FFFFFFFll)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_state_reset: tensor too large");
    return hip_status(ssm::launch_state_reset(src, dst, reset_mask, batch, row_bytes, unit,
                                              threshold, seed, offset,
                                              reinterpret_cast<hipStream_t>(stream)),
                      fn);
}

ssm_status_t ssm_stream_copy(const void* src, void* dst, int64_t bytes, ssm_stream_t stream) {
    const char* fn = "ssm_stream_copy";
    if (bytes < 0) return fail(SSM_ERR_INVALID_ARG, "ssm_stream_copy: need bytes >= 0");
    ssm_status_t st = check_ptrs(fn, {{"src", src, bytes > 0, 1}, {"dst", dst, bytes > 0, 1}});
    if (st != SSM_OK) return st;
    if (bytes == 0) return ok();
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + static_cast<uintptr_t>(bytes) && d0 < s0 + static_cast<uintptr_t>(bytes))
        return fail(SSM_ERR_INVALID_ARG, "ssm_stream_copy: src and dst overlap");
    return hip_status(ssm::launch_stream_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream)), fn);
}

ssm_status_t ssm_timing_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = enable != 0;
    return ok();
}

ssm_status_t ssm_timing_read(double* total_ms, int64_t* launches) {
    if (!total_ms || !launches) return fail(SSM_ERR_INVALID_ARG, "ssm_timing_read: NULL output");
    std::vector<EventPair> evs;
    {
        std::lock_guard<std::mutex> lk(g_tmu);
        evs.swap(g_events);
    }
    double sum = 0.0;
    hipError_t err = hipSuccess;
    for (auto& pr : evs) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(pr.e1);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.e0, pr.e1);
        if (e != hipSuccess && err == hipSuccess) err = e;
        sum += ms;
    }
    {
        std::lock_guard<std::mutex> lk(g_tmu);
        g_spare.insert(g_spare.end(), evs.begin(), evs.end());
    }
    *total_ms = sum;
    *launches = static_cast<int64_t>(evs.size());
    return hip_status(err, "ssm_timing_read");
}

}  // extern "C"
