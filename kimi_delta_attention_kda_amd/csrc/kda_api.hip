// kda_api.hip -- extern "C" entry points of libkda (see include/kda.h):
// argument validation on the host, then kernel launches on the caller's
// stream.  No device allocation and no synchronisation.  Library state lives
// in two device-memory variables, each existing once per GPU: the error word
// (kernels set it when they meet an invalid slot index in device memory;
// kda_device_check reads and clears it) and the static scratch array that
// kda_chunk_fwd_noalloc uses as its workspace.
#include <stdint.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The device error word: one int per GPU (a __device__ variable exists once per
// device the library runs on).  Its address is looked up once per device.
__device__ int g_kda_device_errors;

constexpr int kMaxDevices = 64;
std::mutex g_err_mutex;
int *g_err_ptr[kMaxDevices] = {};

hipError_t error_word(int **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_err_mutex);
    if (!g_err_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_kda_device_errors));
        if (e != hipSuccess) return e;
        g_err_ptr[dev] = static_cast<int *>(p);
    }
    *out = g_err_ptr[dev];
    return hipSuccess;
}

// The workspace of kda_chunk_fwd_noalloc: a fixed array in device memory, one
// per GPU the library runs on, held until the process ends.  Host code never
// uses the array's name as an address (on the host it names a stand-in): it
// takes each device's address once, with hipGetSymbolAddress, and passes that.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_ptr(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Chunk rows of a prefill (sum over sequences of ceil(len / 16)): exact for
// dense input, an upper bound for packed input (whose lengths live in device
// memory): each sequence adds at most one partial chunk.
long long chunk_rows(int B, int T, int n_seq, bool packed)
{
    if (!packed) return (long long)B * ((T + 15) / 16);
    return (long long)(T + 15) / 16 + n_seq;
}

}  // namespace

extern "C" {

const char *kda_status_str(int status)
{
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration (head dims, chunk size or dtype)";
    case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_ERR_HIP: return "HIP launch error";
    case KDA_ERR_SLOT: return "a kernel met a pool slot index >= P (treated as a pad row)";
    case KDA_ERR_SCRATCH: return "the call needs more workspace than the static scratch (KDA_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
    }
}

// Shared body of kda_chunk_fwd and kda_chunk_fwd_pool (state_idx: NULL for the
// dense-state form; then h0 / h_T rows are sequences).
static int chunk_fwd_impl(const void *q, const void *k, const void *v, const void *g_raw,
                          const void *beta_raw, const float *A_log, const float *dt_bias,
                          const float *h0, const int32_t *state_idx, const int32_t *cu_seqlens,
                          int chunk, void *o, float *h_T, float *h_chunks, int B, int T, int H, int dk,
                          int dv, int n_seq, int P, float scale, kda_dtype dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    if (chunk != 16) return KDA_ERR_UNSUPPORTED;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
    if (dtype == KDA_F32 && dk != 64) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H <= 0 || n_seq < 0) return KDA_ERR_SHAPE;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_SHAPE;
    } else if (n_seq != B) {
        return KDA_ERR_SHAPE;
    }
    const long long tokens = cu_seqlens ? (long long)T : (long long)B * T;
    if (tokens * H * (dk > dv ? dk : dv) > 0x7fffffffLL * 8) return KDA_ERR_SHAPE;
    if ((long long)n_seq * H * 2 > 0x7fffffffLL) return KDA_ERR_SHAPE;
    if (!A_log || !dt_bias) return KDA_ERR_NULL;
    if (n_seq > 0 && tokens > 0 && (!q || !k || !v || !g_raw || !beta_raw || !o)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, o, h_T, h_chunks, cu_seqlens, state_idx,
                          workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    if (n_seq == 0) return KDA_OK;

    kda::FwdArgs a;
    if (error_word(&a.err) != hipSuccess) return KDA_ERR_HIP;
    a.q = q; a.k = k; a.v = v; a.g_raw = g_raw; a.beta_raw = beta_raw;
    a.A_log = A_log; a.dt_bias = dt_bias; a.h0 = h0; a.state_idx = state_idx; a.cu_seqlens = cu_seqlens;
    a.o = o; a.h_T = h_T; a.h_chunks = h_chunks; a.T = T; a.H = H; a.n_seq = n_seq; a.P = P;
    a.scale = scale;
    const long long rows = chunk_rows(B, T, n_seq, cu_seqlens != nullptr);
    const hipError_t e = dtype == KDA_BF16 ? kda::launch_fwd_bf16(a, dk, dv, workspace, workspace_bytes, rows, stream)
                                           : kda::launch_fwd_f32(a, dk, dv, stream);
    if (e == hipErrorInvalidValue) return KDA_ERR_UNSUPPORTED;
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int n_seq, int packed)
{
    if (B < 0 || T < 0 || H <= 0 || n_seq < 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return 0;
    return kda::fwd_workspace_bytes(dk, chunk_rows(B, T, n_seq, packed != 0), H);
}

int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g_raw,
                  const void *beta_raw, const float *A_log, const float *dt_bias,
                  const float *h0, const int32_t *cu_seqlens, int chunk, void *o, float *h_T,
                  int B, int T, int H, int dk, int dv, int n_seq, float scale,
                  kda_dtype dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return chunk_fwd_impl(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, nullptr, cu_seqlens, chunk, o,
                          h_T, nullptr, B, T, H, dk, dv, n_seq, 0, scale, dtype, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *g_raw,
                          const void *beta_raw, const float *A_log, const float *dt_bias,
                          const float *h0, const int32_t *cu_seqlens, int chunk, void *o, float *h_T,
                          int B, int T, int H, int dk, int dv, int n_seq, float scale,
                          kda_dtype dtype, hipStream_t stream)
{
    void *ws = nullptr;
    size_t ws_bytes = 0;
    // the bf16 form takes its workspace from the static scratch when it would run
    // in two passes; invalid sizes fall through to kda_chunk_fwd's own checks
    bool sane = chunk == 16 && dtype == KDA_BF16 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128) &&
                B >= 0 && T >= 0 && H > 0 && n_seq > 0 && (long long)n_seq * H * 2 <= 0x7fffffffLL &&
                (cu_seqlens ? B == 1 : n_seq == B) &&
                q && k && v && g_raw && beta_raw && o && A_log && dt_bias;
    const void *ptrs[] = {q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, o, h_T, cu_seqlens};
    for (const void *p : ptrs) sane = sane && (!p || aligned16(p));
    if (sane) {
        bool two = false;
        if (kda::fwd_two_pass_eligible((long long)n_seq * H, &two) != hipSuccess) return KDA_ERR_HIP;
        if (two) {
            const size_t need = kda::fwd_workspace_bytes(dk, chunk_rows(B, T, n_seq, cu_seqlens != nullptr), H);
            if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
            if (scratch_ptr(&ws) != hipSuccess) return KDA_ERR_HIP;
            ws_bytes = KDA_NOALLOC_SCRATCH_BYTES;
        }
    }
    return chunk_fwd_impl(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, nullptr, cu_seqlens, chunk, o,
                          h_T, nullptr, B, T, H, dk, dv, n_seq, 0, scale, dtype, ws, ws_bytes, stream);
}

int kda_chunk_fwd_states(const void *q, const void *k, const void *v, const void *g_raw,
                         const void *beta_raw, const float *A_log, const float *dt_bias,
                         const float *h0, const int32_t *cu_seqlens, int chunk, void *o, float *h_T,
                         float *h_chunks, int B, int T, int H, int dk, int dv, int n_seq, float scale,
                         kda_dtype dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (n_seq > 0 && T > 0 && !h_chunks) return KDA_ERR_NULL;
    return chunk_fwd_impl(q, k, v, g_raw, beta_raw, A_log, dt_bias, h0, nullptr, cu_seqlens, chunk, o,
                          h_T, h_chunks, B, T, H, dk, dv, n_seq, 0, scale, dtype, workspace, workspace_bytes,
                          stream);
}

int kda_chunk_fwd_pool(const void *q, const void *k, const void *v, const void *g_raw,
                       const void *beta_raw, const float *A_log, const float *dt_bias,
                       float *state_pool, const int32_t *state_idx, const int32_t *cu_seqlens,
                       int chunk, void *o, int B, int T, int H, int dk, int dv, int n_seq, int P,
                       float scale, kda_dtype dtype, void *workspace, size_t workspace_bytes,
                       hipStream_t stream)
{
    if (P <= 0) return KDA_ERR_SHAPE;
    if (n_seq > 0 && (!state_pool || !state_idx)) return KDA_ERR_NULL;
    if ((long long)P * H > 0x7fffffffLL) return KDA_ERR_SHAPE;
    // the slots double as h0 (read when a sequence starts) and h_T (written when it
    // ends); each (sequence, head, slab) is read and written by the same workgroup
    return chunk_fwd_impl(q, k, v, g_raw, beta_raw, A_log, dt_bias, state_pool, state_idx, cu_seqlens,
                          chunk, o, state_pool, nullptr, B, T, H, dk, dv, n_seq, P, scale, dtype, workspace,
                          workspace_bytes, stream);
}

int kda_chunk_o(const void *q, const void *k, const void *v, const void *g_raw, const void *beta_raw,
                const float *A_log, const float *dt_bias, const float *h_chunks,
                const int32_t *cu_seqlens, void *o, int B, int T, int H, int dk, int dv, int n_seq,
                int n_chunks, float scale, kda_dtype dtype, hipStream_t stream)
{
    if (dtype != KDA_BF16 || dk != 128 || dv != 128) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H <= 0 || n_seq < 0 || n_chunks < 0) return KDA_ERR_SHAPE;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_SHAPE;
    } else {
        if (n_seq != B) return KDA_ERR_SHAPE;
        if ((long long)n_chunks != (long long)B * ((T + 15) / 16)) return KDA_ERR_SHAPE;
    }
    if ((long long)n_chunks * H > 0x7fffffffLL) return KDA_ERR_SHAPE;
    if (n_chunks == 0 || n_seq == 0) return KDA_OK;
    if (!q || !k || !v || !g_raw || !beta_raw || !A_log || !dt_bias || !h_chunks || !o) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g_raw, beta_raw, A_log, dt_bias, h_chunks, cu_seqlens, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    kda::ChunkOArgs a;
    a.q = q; a.k = k; a.v = v; a.g_raw = g_raw; a.beta_raw = beta_raw;
    a.A_log = A_log; a.dt_bias = dt_bias; a.h_chunks = h_chunks; a.cu_seqlens = cu_seqlens;
    a.o = o; a.T = T; a.H = H; a.n_seq = n_seq; a.scale = scale;
    const hipError_t e = kda::launch_chunk_o(a, n_chunks, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_backward_workspace_bytes(int n_seq, int H, int dk, int dv, int64_t total_tokens)
{
    if (n_seq < 0 || H <= 0 || dk != 128 || dv != 128 || total_tokens < 0) return 0;
    return kda::bwd_workspace_bytes(n_seq, H, total_tokens);
}

int kda_backward(const void *q, const void *k, const void *v, const void *g_raw, const void *beta_raw,
                 const float *A_log, const float *dt_bias, const float *h_chunks,
                 const int32_t *cu_seqlens, const void *do_, const float *dh_T, void *dq, void *dk,
                 void *dv, void *dg_raw, void *dbeta_raw, float *dA_log, float *ddt_bias, float *dh0,
                 void *workspace, size_t workspace_bytes, int B, int T, int H, int dk_, int dv_,
                 int n_seq, float scale, kda_dtype dtype, hipStream_t stream)
{
    // the stored states come from the bf16 d = 128 forward (fp32 activations are built for dk = 64 only)
    if (dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk_ != 128 || dv_ != 128) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H <= 0 || n_seq < 0) return KDA_ERR_SHAPE;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_SHAPE;
    } else if (n_seq != B) {
        return KDA_ERR_SHAPE;
    }
    const long long tokens = cu_seqlens ? (long long)T : (long long)B * T;
    if (tokens * H * 128 > 0x7fffffffLL * 8) return KDA_ERR_SHAPE;
    if ((long long)n_seq * H > 0x7fffffffLL) return KDA_ERR_SHAPE;
    if (n_seq == 0) return KDA_OK;
    if (!A_log || !dt_bias || !workspace) return KDA_ERR_NULL;
    if (tokens > 0 && (!q || !k || !v || !g_raw || !beta_raw || !h_chunks || !do_ || !dq || !dk || !dv ||
                       !dg_raw || !dbeta_raw))
        return KDA_ERR_NULL;
    if (workspace_bytes < kda::bwd_workspace_bytes(n_seq, H, tokens)) return KDA_ERR_SHAPE;
    const void *ptrs[] = {q, k, v, g_raw, beta_raw, A_log, dt_bias, h_chunks, cu_seqlens, do_, dh_T,
                          dq, dk, dv, dg_raw, dbeta_raw, dA_log, ddt_bias, dh0, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    kda::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g_raw = g_raw; a.beta_raw = beta_raw; a.do_ = do_;
    a.A_log = A_log; a.dt_bias = dt_bias; a.h_chunks = h_chunks; a.dh_T = dh_T; a.cu_seqlens = cu_seqlens;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg_raw = dg_raw; a.dbeta_raw = dbeta_raw;
    a.dA_log = dA_log; a.ddt_bias = ddt_bias; a.dh0 = dh0;
    a.work = workspace;
    a.T = T; a.H = H; a.n_seq = n_seq; a.T_all = tokens; a.scale = scale;
    const hipError_t e = kda::launch_bwd(a, dtype == KDA_BF16 ? 1 : 0, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_device_check(hipStream_t stream)
{
    int *err = nullptr;
    if (error_word(&err) != hipSuccess) return KDA_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
    int h = 0;
    if (hipMemcpy(&h, err, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return KDA_ERR_HIP;
    if (h) {
        const int zero = 0;
        if (hipMemcpy(err, &zero, sizeof(int), hipMemcpyHostToDevice) != hipSuccess) return KDA_ERR_HIP;
    }
    return (h & KDA_DEVERR_SLOT) ? KDA_ERR_SLOT : KDA_OK;
}

int kda_decode_step(const void *qkv, const void *a, const void *b, const float *A_log,
                    const float *dt_bias, float *state_pool, const int32_t *state_idx, void *o,
                    int B, int H, int HV, int K, int V, int P, float scale, int flags,
                    hipStream_t stream)
{
    if (K != 128 || V != 128) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || H <= 0 || HV <= 0 || HV % H != 0 || P < 0) return KDA_ERR_SHAPE;
    if ((long long)B * HV > 0x7fffffffLL) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    if (!qkv || !a || !b || !A_log || !dt_bias || !state_pool || !state_idx || !o) return KDA_ERR_NULL;
    const void *ptrs[] = {qkv, a, b, A_log, dt_bias, state_pool, state_idx, o};
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    int *err = nullptr;
    if (error_word(&err) != hipSuccess) return KDA_ERR_HIP;
    const hipError_t e = kda::launch_decode(
        static_cast<const uint16_t *>(qkv), static_cast<const uint16_t *>(a),
        static_cast<const uint16_t *>(b), A_log, dt_bias, state_pool, state_idx,
        static_cast<uint16_t *>(o), B, H, HV, P, scale, flags & KDA_DECODE_L2NORM, err, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_extend(const void *qkv, const void *a, const void *b, const float *A_log,
                      const float *dt_bias, float *state_pool, const int32_t *state_idx, void *o,
                      int B, int T, int H, int HV, int K, int V, int P, float scale, int flags,
                      hipStream_t stream)
{
    if (K != 128 || V != 128) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || HV % H != 0 || P < 0) return KDA_ERR_SHAPE;
    if ((long long)B * HV > 0x7fffffffLL) return KDA_ERR_SHAPE;
    if ((long long)B * T * (2LL * H * K + (long long)HV * V) > 0x7fffffffLL * 8) return KDA_ERR_SHAPE;
    if (B == 0 || T == 0) return KDA_OK;
    if (!qkv || !a || !b || !A_log || !dt_bias || !state_pool || !state_idx || !o) return KDA_ERR_NULL;
    const void *ptrs[] = {qkv, a, b, A_log, dt_bias, state_pool, state_idx, o};
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    int *err = nullptr;
    if (error_word(&err) != hipSuccess) return KDA_ERR_HIP;
    const hipError_t e = kda::launch_extend(
        static_cast<const uint16_t *>(qkv), static_cast<const uint16_t *>(a),
        static_cast<const uint16_t *>(b), A_log, dt_bias, state_pool, state_idx,
        static_cast<uint16_t *>(o), B, T, H, HV, P, scale, flags & KDA_DECODE_L2NORM, err, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_conv_decode_step(const void *mixed_qkv, void *conv_state, const void *conv_weight,
                         const void *conv_bias, const void *a, const void *b, const float *A_log,
                         const float *dt_bias, float *state_pool, const int32_t *state_idx, void *o,
                         int B, int H, int HV, int K, int V, int W, int P, float scale, int flags,
                         hipStream_t stream)
{
    if (K != 128 || V != 128 || W < 2 || W > 4) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || H <= 0 || HV <= 0 || HV % H != 0 || P < 0) return KDA_ERR_SHAPE;
    if ((long long)B * HV > 0x7fffffffLL) return KDA_ERR_SHAPE;
    // the conv outputs of one workgroup (q, k and HV/H value heads, fp32) sit in LDS
    if (sizeof(float) * (2LL * K + (long long)(HV / H) * V) > 65536) return KDA_ERR_UNSUPPORTED;
    if (B == 0) return KDA_OK;
    if (!mixed_qkv || !conv_state || !conv_weight || !a || !b || !A_log || !dt_bias || !state_pool ||
        !state_idx || !o)
        return KDA_ERR_NULL;
    const void *ptrs[] = {mixed_qkv, conv_state, conv_weight, conv_bias, a, b, A_log, dt_bias,
                          state_pool, state_idx, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    int *err = nullptr;
    if (error_word(&err) != hipSuccess) return KDA_ERR_HIP;
    const hipError_t e = kda::launch_conv_decode(
        static_cast<const uint16_t *>(mixed_qkv), static_cast<uint16_t *>(conv_state),
        static_cast<const uint16_t *>(conv_weight), static_cast<const uint16_t *>(conv_bias),
        static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(b), A_log, dt_bias, state_pool,
        state_idx, static_cast<uint16_t *>(o), B, H, HV, W, P, scale, flags & KDA_DECODE_L2NORM, err, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
