// fa_api.hip -- the C ABI declared in include/fa.h: argument checks, kernel
// selection and launch-error reporting.  Every check happens on the host
// before any launch; nothing here allocates device memory.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa.h"
#include "fa_kernels.h"
#include "fa_probe.h"
#include "fa_testing.h"

namespace {

thread_local char g_last_hip_error[256] = "";

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

fa_status from_hip(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return FA_ERR_HIP;
}

constexpr long long kMaxGridX = 0x7fffffffLL;
constexpr long long kMaxGridYZ = 65535;
constexpr long long kMaxElems = 1LL << 46;   // far beyond 288 GB of bf16
constexpr long long kMaxSliceBytes = (1LL << 31) - 256;   // per (b, h) slice
constexpr long long kMaxSoftmaxCols = 1LL << 30;         // chunk indices stay 32-bit

}  // namespace

namespace fa {

// Compute units of the current device, looked up once per device.  A failed
// query falls back to 256 (MI355X) and clears the runtime's last error, so the
// launch that follows reports only its own status.
int device_cu_count() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return 256;
    }
    int v = cache[dev].load(std::memory_order_relaxed);
    if (!v) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
            (void)hipGetLastError();
            v = 256;
        }
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

}  // namespace fa

extern "C" {

const char *fa_status_str(fa_status status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        case FA_ERR_SCRATCH_LIMIT: return "FA_ERR_SCRATCH_LIMIT";
    }
    return "FA_ERR_UNKNOWN";
}

const char *fa_last_hip_error(void) { return g_last_hip_error; }

fa_status fa_forward(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                     int H, int N, int Nk, int d, float scale, int causal,
                     const int32_t *key_lens, fa_dtype dtype, void *stream) {
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || N < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype == FA_BF16 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_F32 && d > 256) return FA_ERR_UNSUPPORTED;
    if (scale <= 0.f) return FA_ERR_UNSUPPORTED;
    const long long rows = (long long)B * H * N;
    if (rows == 0) return FA_OK;
    if ((long long)B * H * (long long)(N > Nk ? N : Nk) * d > kMaxElems) return FA_ERR_INVALID_ARG;
    // one (b, h) slice of Q/O or K/V is addressed with 32-bit byte offsets
    const long long esz = dtype == FA_BF16 ? 2 : 4;
    if ((long long)(N > Nk ? N : Nk) * d * esz > kMaxSliceBytes) return FA_ERR_INVALID_ARG;
    if (!Q || !O || !LSE) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!K || !V)) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(O) || !aligned4(LSE)) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!aligned16(K) || !aligned16(V))) return FA_ERR_INVALID_ARG;
    if (key_lens && !aligned4(key_lens)) return FA_ERR_INVALID_ARG;
    const int rows_per_block = dtype == FA_BF16 ? 128 : 64;
    const long long nblocks = (long long)B * H * ((N + rows_per_block - 1) / rows_per_block);
    if (nblocks > kMaxGridX) return FA_ERR_INVALID_ARG;

    fa::FwdArgs a{Q, K, V, O, LSE, key_lens, B, H, N, Nk, d, scale, causal};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return from_hip(dtype == FA_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
    if (B < 0 || H < 0 || d < 0 || num_splits < 1) return 0;
    return (size_t)B * (size_t)H * (size_t)num_splits * ((size_t)d + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by the two decode entry points (everything but the workspace).
fa_status check_decode(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                       int H, int Nk, int d, float scale, const int32_t *key_lens, int num_splits,
                       fa_dtype dtype) {
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (num_splits < 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype == FA_BF16 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_F32 && d > 256) return FA_ERR_UNSUPPORTED;
    if (num_splits > 256) return FA_ERR_UNSUPPORTED;
    if (scale <= 0.f) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return FA_OK;
    if ((long long)B * H * (long long)Nk * d > kMaxElems) return FA_ERR_INVALID_ARG;
    if ((long long)Nk * d * (dtype == FA_BF16 ? 2 : 4) > kMaxSliceBytes) return FA_ERR_INVALID_ARG;
    if (B > kMaxGridYZ || H > kMaxGridYZ || (long long)B * H > kMaxGridX) return FA_ERR_INVALID_ARG;
    if (!Q || !O || !LSE) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!K || !V)) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(O) || !aligned4(LSE)) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!aligned16(K) || !aligned16(V))) return FA_ERR_INVALID_ARG;
    if (key_lens && !aligned4(key_lens)) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_decode_splitkv(const void *Q, const void *K, const void *V, void *O, float *LSE,
                            int B, int H, int Nk, int d, float scale, const int32_t *key_lens,
                            int num_splits, void *workspace, size_t workspace_bytes,
                            fa_dtype dtype, void *stream) {
    const fa_status st = check_decode(Q, K, V, O, LSE, B, H, Nk, d, scale, key_lens, num_splits, dtype);
    if (st != FA_OK || (long long)B * H == 0) return st;
    if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
    if (workspace_bytes < fa_decode_workspace_bytes(B, H, d, num_splits)) return FA_ERR_INVALID_ARG;

    fa::DecodeArgs a{Q, K, V, O, LSE, key_lens, B, H, Nk, d, scale, num_splits,
                     static_cast<float *>(workspace)};
    return from_hip(fa::launch_decode(a, dtype == FA_BF16, static_cast<hipStream_t>(stream)));
}

size_t fa_decode_scratch_bytes(void) { return fa::kDecodeScratchBytes; }

fa_status fa_decode_splitkv_noalloc(const void *Q, const void *K, const void *V, void *O, float *LSE,
                                    int B, int H, int Nk, int d, float scale,
                                    const int32_t *key_lens, int num_splits, fa_dtype dtype,
                                    void *stream) {
    const fa_status st = check_decode(Q, K, V, O, LSE, B, H, Nk, d, scale, key_lens, num_splits, dtype);
    if (st != FA_OK || (long long)B * H == 0) return st;
    // sizes are checked before the device is touched
    if (fa_decode_workspace_bytes(B, H, d, num_splits) > fa::kDecodeScratchBytes)
        return FA_ERR_SCRATCH_LIMIT;
    void *scr = nullptr;
    const hipError_t e = fa::decode_scratch(&scr);
    if (e != hipSuccess) return from_hip(e);
    fa::DecodeArgs a{Q, K, V, O, LSE, key_lens, B, H, Nk, d, scale, num_splits,
                     static_cast<float *>(scr)};
    return from_hip(fa::launch_decode(a, dtype == FA_BF16, static_cast<hipStream_t>(stream)));
}

size_t fa_softmax_workspace_bytes(int64_t rows, int64_t cols, fa_dtype dtype) {
    if (rows < 0 || cols < 0 || (dtype != FA_F32 && dtype != FA_BF16)) return 0;
    if ((long long)rows * (long long)cols > kMaxElems || cols > kMaxSoftmaxCols) return 0;
    return fa::softmax_workspace_bytes(rows, cols, dtype == FA_BF16);
}

fa_status fa_softmax(const void *X, void *Y, float *LSE, int64_t rows, int64_t cols,
                     fa_dtype dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return FA_ERR_INVALID_ARG;
    if (rows == 0) return FA_OK;
    if (cols > kMaxSoftmaxCols || (long long)rows * (long long)cols > kMaxElems)
        return FA_ERR_INVALID_ARG;
    if (rows > kMaxGridX) return FA_ERR_INVALID_ARG;
    if (!LSE || !aligned4(LSE)) return FA_ERR_INVALID_ARG;
    if (cols > 0 && (!X || !aligned16(X))) return FA_ERR_INVALID_ARG;
    if (Y && !aligned16(Y)) return FA_ERR_INVALID_ARG;
    const size_t need = fa::softmax_workspace_bytes(rows, cols, dtype == FA_BF16);
    if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return FA_ERR_INVALID_ARG;
    if (cols == 0) Y = nullptr;   // nothing to write but lse = -inf
    fa::SoftmaxArgs a{X, Y, LSE, rows, cols, workspace};
    return from_hip(fa::launch_softmax(a, dtype == FA_BF16, static_cast<hipStream_t>(stream)));
}

size_t fa_forward_v1_workspace_bytes(int B, int H, int N, int d) {
    if (B < 0 || H < 0 || N < 0 || d < 0) return 0;
    return fa::forward_v1_workspace_bytes(B, H, N, d);
}

fa_status fa_forward_v1(const void *Q, const void *K, const void *V, void *O, float *LSE, int B,
                        int H, int N, int Nk, int d, float scale, int causal,
                        const int32_t *key_lens, void *workspace, size_t workspace_bytes,
                        fa_dtype dtype, void *stream) {
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || N < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if (scale <= 0.f) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * N == 0) return FA_OK;
    if ((long long)B * H * (long long)(N > Nk ? N : Nk) * d > kMaxElems) return FA_ERR_INVALID_ARG;
    if ((long long)(N > Nk ? N : Nk) * d * 4 > kMaxSliceBytes) return FA_ERR_INVALID_ARG;
    if ((long long)B * H > kMaxGridX) return FA_ERR_INVALID_ARG;
    if (!Q || !O || !LSE) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!K || !V)) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(O) || !aligned4(LSE)) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!aligned16(K) || !aligned16(V))) return FA_ERR_INVALID_ARG;
    if (key_lens && !aligned4(key_lens)) return FA_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) ||
        workspace_bytes < fa::forward_v1_workspace_bytes(B, H, N, d))
        return FA_ERR_INVALID_ARG;
    fa::FwdArgs a{Q, K, V, O, LSE, key_lens, B, H, N, Nk, d, scale, causal};
    return from_hip(fa::launch_fwd_v1(a, workspace, static_cast<hipStream_t>(stream)));
}

size_t fa_backward_workspace_bytes(int B, int H, int N) {
    if (B < 0 || H < 0 || N < 0) return 0;
    return fa::backward_workspace_bytes(B, H, N);
}

fa_status fa_backward(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                      const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int N, int Nk,
                      int d, float scale, int causal, const int32_t *key_lens, void *workspace,
                      size_t workspace_bytes, fa_dtype dtype, void *stream) {
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || N < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype == FA_BF16 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_F32 && d > 256) return FA_ERR_UNSUPPORTED;
    if (scale <= 0.f) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0 || (N == 0 && Nk == 0)) return FA_OK;
    if ((long long)B * H * (long long)(N > Nk ? N : Nk) * d > kMaxElems) return FA_ERR_INVALID_ARG;
    if ((long long)(N > Nk ? N : Nk) * d * (dtype == FA_BF16 ? 2 : 4) > kMaxSliceBytes)
        return FA_ERR_INVALID_ARG;
    if (N > 0 && (!Q || !O || !dO || !LSE || !dQ)) return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!K || !V || !dK || !dV)) return FA_ERR_INVALID_ARG;
    if (N > 0 && (!aligned16(Q) || !aligned16(O) || !aligned16(dO) || !aligned16(dQ) ||
                  !aligned4(LSE)))
        return FA_ERR_INVALID_ARG;
    if (Nk > 0 && (!aligned16(K) || !aligned16(V) || !aligned16(dK) || !aligned16(dV)))
        return FA_ERR_INVALID_ARG;
    if (key_lens && !aligned4(key_lens)) return FA_ERR_INVALID_ARG;
    const size_t need = fa::backward_workspace_bytes(B, H, N);
    if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return FA_ERR_INVALID_ARG;
    // the smallest workgroups hold 16 rows (fp32, d > 128)
    const long long blocks = (long long)B * H * (((N > Nk ? N : Nk) + 15) / 16);
    if (blocks > kMaxGridX) return FA_ERR_INVALID_ARG;
    fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, key_lens, B, H, N, Nk, d, scale, causal, workspace};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return from_hip(dtype == FA_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f32(a, s));
}

void fa_testing_set_softmax_spin_limit(int limit) { fa::set_softmax_spin_limit(limit); }

void fa_testing_set_rescale_rule(int rule) { fa::set_rescale_rule(rule); }

fa_status fa_probe_mfma(float *sink, int blocks, int iters, void *stream) {
    if (!sink || !aligned4(sink) || blocks < 1 || blocks > kMaxGridX || iters < 1) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_probe_mfma(sink, blocks, iters, static_cast<hipStream_t>(stream)));
}

fa_status fa_probe_read(const void *src, size_t bytes, uint32_t *sink, int blocks, void *stream) {
    if ((bytes > 0 && (!src || !aligned16(src))) || bytes % 16 != 0 || !sink || !aligned4(sink) ||
        blocks < 1 || blocks > kMaxGridX)
        return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_probe_read(src, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

fa_status fa_probe_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream) {
    if (bytes % 16 != 0 || blocks < 1 || blocks > kMaxGridX) return FA_ERR_INVALID_ARG;
    if (bytes == 0) return FA_OK;
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return FA_ERR_INVALID_ARG;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return FA_ERR_INVALID_ARG;   // overlapping ranges
    return from_hip(fa::launch_probe_copy(src, dst, bytes, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
