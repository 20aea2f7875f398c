// lion_abi.hip -- the extern "C" boundary of the LION attention library.
//
// Every argument is checked on the host before any HIP call; a rejected call touches no buffer
// and enqueues nothing.  Valid calls are handed to the launchers of the three forms.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "lion_attn.h"
#include "lion_internal.h"

namespace {

constexpr long long kMaxL = 1 << 22;          // positions per sequence
constexpr long long kMaxRows = 1LL << 31;     // B * H * L (row indices stay in int range)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool d_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool c_supported(int C) { return C == 16 || C == 32 || C == 64 || C == 128 || C == 256; }
// a chunk's query tiles must fit one pass of the chunk kernel's waves (256 rows, 128 for d = 128)
bool c_supported_for(int C, int d) { return c_supported(C) && (d < 128 || C <= 128); }

// Shared checks of the three entry points; returns LION_OK or a negative status.
int check_common(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, float eps,
                 int B, int H, int L, int d, int dtype, const void *y, int y_dtype, const float *den_out) {
    if (!q || !k || !v || !y) return LION_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return LION_ERR_INVALID;
    if (den_out && !aligned16(den_out)) return LION_ERR_INVALID;
    if (mask_kind & ~(3 | LION_CAUSAL | LION_FP32_ARITH)) return LION_ERR_INVALID;
    const int kind = mask_kind & 3;
    if (kind != LION_MASK_LIT && kind != LION_MASK_D && kind != LION_MASK_S) return LION_ERR_INVALID;
    if (kind == LION_MASK_LIT ? log_lambda != nullptr : log_lambda == nullptr) return LION_ERR_INVALID;
    if (log_lambda && !aligned16(log_lambda)) return LION_ERR_INVALID;
    if (!(eps >= 0.f) || !isfinite(eps)) return LION_ERR_INVALID;
    if (B < 1 || H < 1 || L < 1 || d < 1) return LION_ERR_INVALID;
    if ((long long)L > kMaxL || (long long)B * H * L > kMaxRows) return LION_ERR_INVALID;
    if (dtype != LION_DTYPE_F32 && dtype != LION_DTYPE_BF16) return LION_ERR_INVALID;
    if (y_dtype != LION_DTYPE_F32 && y_dtype != LION_DTYPE_BF16) return LION_ERR_INVALID;
    if (!d_supported(d)) return LION_ERR_UNSUPPORTED;
    if (dtype == LION_DTYPE_F32 && y_dtype != LION_DTYPE_F32) return LION_ERR_UNSUPPORTED;
    return LION_OK;
}

lion::AttnArgs make_args(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind,
                         float eps, int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out) {
    lion::AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_lambda = log_lambda;
    a.kind = mask_kind & 3;
    a.causal = (mask_kind & LION_CAUSAL) != 0;
    a.eps = eps;
    a.B = B;
    a.H = H;
    a.L = L;
    a.d = d;
    a.in_bf16 = dtype == LION_DTYPE_BF16;
    a.fp32c = !a.in_bf16 || (mask_kind & LION_FP32_ARITH) != 0;
    a.y = y;
    a.out_bf16 = y_dtype == LION_DTYPE_BF16;
    a.den_out = den_out;
    a.order = nullptr;
    a.C = 0;
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    return a;
}

int status_of(hipError_t e) { return e == hipSuccess ? LION_OK : LION_ERR_HIP; }

}  // namespace

extern "C" {

int lion_attn_full(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, float eps,
                   int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out, void *stream) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (rc != LION_OK) return rc;
    lion::AttnArgs a = make_args(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (!lion::plan_full(a).ok) return LION_ERR_UNSUPPORTED;
    return status_of(lion::launch_full(a, reinterpret_cast<hipStream_t>(stream)));
}

int lion_attn_full2(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, float eps,
                    const int *order, int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out,
                    void *stream) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (rc != LION_OK) return rc;
    if (!order || !aligned16(order)) return LION_ERR_INVALID;
    if (mask_kind & (LION_CAUSAL | LION_FP32_ARITH)) return LION_ERR_UNSUPPORTED;
    lion::AttnArgs a = make_args(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    a.order = order;
    if (!lion::plan_full(a).ok) return LION_ERR_UNSUPPORTED;
    return status_of(lion::launch_full(a, reinterpret_cast<hipStream_t>(stream)));
}

int lion_attn_chunk(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int C,
                    float eps, int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out,
                    void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (rc != LION_OK) return rc;
    if (C < 1) return LION_ERR_INVALID;
    if (!c_supported_for(C, d)) return LION_ERR_UNSUPPORTED;
    if (workspace && !aligned16(workspace)) return LION_ERR_INVALID;
    lion::AttnArgs a = make_args(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    a.C = C;
    const lion::Plan plan = lion::plan_chunk(a);
    if (!plan.ok) return LION_ERR_UNSUPPORTED;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return LION_ERR_WORKSPACE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return status_of(lion::launch_chunk(a, reinterpret_cast<hipStream_t>(stream)));
}

int lion_attn_chunk2(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int C,
                     float eps, const int *order, int B, int H, int L, int d, int dtype, void *y, int y_dtype,
                     float *den_out, void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (rc != LION_OK) return rc;
    if (!order || !aligned16(order)) return LION_ERR_INVALID;
    if (C < 1) return LION_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return LION_ERR_INVALID;
    if (mask_kind & (LION_CAUSAL | LION_FP32_ARITH)) return LION_ERR_UNSUPPORTED;
    if (!c_supported_for(C, d)) return LION_ERR_UNSUPPORTED;
    lion::AttnArgs a = make_args(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    a.C = C;
    a.order = order;
    const lion::Plan plan = lion::plan_chunk2(a);
    if (!plan.ok) return LION_ERR_UNSUPPORTED;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return LION_ERR_WORKSPACE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return status_of(lion::launch_chunk2(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Scratch of lion_attn_chunk_noalloc: one copy per GPU, allocated with the code object and held until
// the process ends.  In host code `scratch` names a host-side stand-in; the device address of each
// GPU's copy comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoallocScratchBytes = LION_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (nullptr and an error if it cannot be had).
void *device_scratch(int *status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = LION_ERR_HIP;
        return nullptr;
    }
    std::call_once(scratch_once[dev], [dev] {
        void *ptr = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) {
        *status = LION_ERR_HIP;
        return nullptr;
    }
    *status = LION_OK;
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int lion_attn_chunk_noalloc(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int C,
                            float eps, int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out,
                            void *stream) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (rc != LION_OK) return rc;
    if (C < 1) return LION_ERR_INVALID;
    if (!c_supported_for(C, d)) return LION_ERR_UNSUPPORTED;
    lion::AttnArgs a = make_args(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    a.C = C;
    const lion::Plan plan = lion::plan_chunk(a);
    if (!plan.ok) return LION_ERR_UNSUPPORTED;
    if (plan.workspace > kNoallocScratchBytes) return LION_ERR_WORKSPACE;   // beyond the built-in scratch
    if (plan.workspace > 0) {
        a.workspace = device_scratch(&rc);
        if (rc != LION_OK) return rc;
        a.workspace_bytes = kNoallocScratchBytes;
    }
    return status_of(lion::launch_chunk(a, reinterpret_cast<hipStream_t>(stream)));
}

int lion_attn_birnn(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, float eps,
                    int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out, void *workspace,
                    size_t workspace_bytes, void *stream) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    if (rc != LION_OK) return rc;
    if (workspace && !aligned16(workspace)) return LION_ERR_INVALID;
    lion::AttnArgs a = make_args(q, k, v, log_lambda, mask_kind, eps, B, H, L, d, dtype, y, y_dtype, den_out);
    const lion::Plan plan = lion::plan_birnn(a);
    if (!plan.ok) return LION_ERR_UNSUPPORTED;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return LION_ERR_WORKSPACE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return status_of(lion::launch_birnn(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks shared by the two backward entry points; fills `a` (workspace excluded) on success.
int bwd_args(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int B, int H, int L,
             int d, int dtype, const void *y, const float *den, const void *dy, void *dq, void *dk, void *dv,
             int grad_dtype, float *dlog_lambda, const void *workspace, lion::BwdArgs &a) {
    int rc = check_common(q, k, v, log_lambda, mask_kind, 0.f, B, H, L, d, dtype, y, dtype, nullptr);
    if (rc != LION_OK) return rc;
    if (!den || !dy || !dq || !dk || !dv) return LION_ERR_INVALID;
    if (mask_kind & LION_FP32_ARITH) return LION_ERR_UNSUPPORTED;
    if (!aligned16(den) || !aligned16(dy) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return LION_ERR_INVALID;
    const int kind = mask_kind & 3;
    if (kind == LION_MASK_LIT ? dlog_lambda != nullptr : dlog_lambda == nullptr) return LION_ERR_INVALID;
    if (dlog_lambda && !aligned16(dlog_lambda)) return LION_ERR_INVALID;
    if (grad_dtype != LION_DTYPE_F32 && grad_dtype != LION_DTYPE_BF16) return LION_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return LION_ERR_INVALID;
    if (dtype != LION_DTYPE_BF16) return LION_ERR_UNSUPPORTED;
    a = lion::BwdArgs{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_lambda = log_lambda;
    a.kind = kind;
    a.causal = (mask_kind & LION_CAUSAL) != 0;
    a.B = B;
    a.H = H;
    a.L = L;
    a.d = d;
    a.y = y;
    a.dy = dy;
    a.den = den;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.g_bf16 = grad_dtype == LION_DTYPE_BF16;
    a.dll = dlog_lambda;
    return LION_OK;
}

}  // namespace

extern "C" {

int lion_attn_full_bwd(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int B,
                       int H, int L, int d, int dtype, const void *y, const float *den, const void *dy, void *dq,
                       void *dk, void *dv, int grad_dtype, float *dlog_lambda, void *workspace, size_t workspace_bytes,
                       void *stream) {
    lion::BwdArgs a;
    const int rc = bwd_args(q, k, v, log_lambda, mask_kind, B, H, L, d, dtype, y, den, dy, dq, dk, dv, grad_dtype,
                            dlog_lambda, workspace, a);
    if (rc != LION_OK) return rc;
    const lion::Plan plan = lion::plan_full_bwd(a);
    if (!plan.ok) return LION_ERR_UNSUPPORTED;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return LION_ERR_WORKSPACE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return status_of(lion::launch_full_bwd(a, reinterpret_cast<hipStream_t>(stream)));
}

int lion_attn_chunk_bwd(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int C,
                        int B, int H, int L, int d, int dtype, const void *y, const float *den, const void *dy,
                        void *dq, void *dk, void *dv, int grad_dtype, float *dlog_lambda, void *workspace,
                        size_t workspace_bytes, void *stream) {
    lion::BwdArgs a;
    const int rc = bwd_args(q, k, v, log_lambda, mask_kind, B, H, L, d, dtype, y, den, dy, dq, dk, dv, grad_dtype,
                            dlog_lambda, workspace, a);
    if (rc != LION_OK) return rc;
    if (!c_supported(C)) return LION_ERR_UNSUPPORTED;
    a.C = C;
    const lion::Plan plan = lion::plan_chunk_bwd(a);
    if (!plan.ok) return LION_ERR_UNSUPPORTED;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return LION_ERR_WORKSPACE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return status_of(lion::launch_chunk_bwd(a, reinterpret_cast<hipStream_t>(stream)));
}

int lion_selectivity(const void *x, const void *w, const float *bias, int B, int L, int H, int Dm, float *log_lambda,
                     float *key_scale, const void *k, void *k_out, int d, void *stream) {
    if (!x || !w || !bias || !log_lambda) return LION_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w) || !aligned16(bias) || !aligned16(log_lambda)) return LION_ERR_INVALID;
    if (key_scale && !aligned16(key_scale)) return LION_ERR_INVALID;
    if (!k != !k_out) return LION_ERR_INVALID;
    if (k && (!aligned16(k) || !aligned16(k_out) || d < 1)) return LION_ERR_INVALID;
    if (B < 1 || L < 1 || H < 1 || Dm < 1) return LION_ERR_INVALID;
    if ((long long)L > kMaxL || (long long)B * H * L > kMaxRows || (long long)B * L * Dm > (1LL << 40))
        return LION_ERR_INVALID;
    lion::SelArgs a;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.B = B;
    a.L = L;
    a.H = H;
    a.Dm = Dm;
    a.log_lambda = log_lambda;
    a.key_scale = key_scale;
    a.k = k;
    a.k_out = k_out;
    a.d = k ? d : 0;
    if (!lion::plan_selectivity(a).ok) return LION_ERR_UNSUPPORTED;
    return status_of(lion::launch_selectivity(a, reinterpret_cast<hipStream_t>(stream)));
}

size_t lion_attn_workspace_bytes(int form, int B, int H, int L, int d, int C, int dtype) {
    if (B < 1 || H < 1 || L < 1 || !d_supported(d) || (long long)L > kMaxL || (long long)B * H * L > kMaxRows)
        return (size_t)-1;
    if (dtype != LION_DTYPE_F32 && dtype != LION_DTYPE_BF16) return (size_t)-1;
    // the plans depend on sizes, dtype and the mask kind: LION-S is the largest of the kinds for the
    // full and chunkwise forms (LDS), and the RNN form's answer is the largest over the kinds
    lion::AttnArgs a = make_args(nullptr, nullptr, nullptr, nullptr, LION_MASK_S, 0.f, B, H, L, d, dtype, nullptr,
                                 dtype, nullptr);
    lion::Plan plan;
    switch (form) {
    case LION_FORM_FULL: plan = lion::plan_full(a); break;
    case LION_FORM_CHUNK: {
        if (!c_supported_for(C, d)) return (size_t)-1;
        a.C = C;
        plan = lion::plan_chunk(a);
        if (a.in_bf16) {   // bf16 inputs may ask for fp32 arithmetic, whose states are fp32
            a.fp32c = true;
            const lion::Plan pf = lion::plan_chunk(a);
            plan.ok = plan.ok && pf.ok;
            if (pf.workspace > plan.workspace) plan.workspace = pf.workspace;
            a.fp32c = false;
        }
        break;
    }
    case LION_FORM_BIRNN: {
        plan = lion::plan_birnn(a);
        for (int kind : {LION_MASK_LIT, LION_MASK_D}) {
            a.kind = kind;
            const lion::Plan pk = lion::plan_birnn(a);
            plan.ok = plan.ok && pk.ok;
            if (pk.workspace > plan.workspace) plan.workspace = pk.workspace;
        }
        break;
    }
    case LION_FORM_CHUNK2:
        if (!c_supported_for(C, d)) return (size_t)-1;
        a.C = C;
        plan = lion::plan_chunk2(a);
        break;
    case LION_FORM_FULL_BWD: {
        if (dtype != LION_DTYPE_BF16) return (size_t)-1;
        lion::BwdArgs b{};
        b.kind = LION_MASK_S;
        b.B = B;
        b.H = H;
        b.L = L;
        b.d = d;
        plan = lion::plan_full_bwd(b);
        break;
    }
    case LION_FORM_CHUNK_BWD: {
        if (dtype != LION_DTYPE_BF16) return (size_t)-1;
        lion::BwdArgs b{};
        b.kind = LION_MASK_S;
        b.B = B;
        b.H = H;
        b.L = L;
        b.d = d;
        b.C = C;
        plan = lion::plan_chunk_bwd(b);
        break;
    }
    default: return (size_t)-1;
    }
    return plan.ok ? plan.workspace : (size_t)-1;
}

const char *lion_status_str(int status) {
    switch (status) {
    case LION_OK: return "ok";
    case LION_ERR_INVALID: return "invalid argument";
    case LION_ERR_UNSUPPORTED: return "unsupported combination";
    case LION_ERR_WORKSPACE: return "workspace too small";
    case LION_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int lion_attn_abi_version(void) { return LION_ATTN_ABI_VERSION; }

}  // extern "C"
