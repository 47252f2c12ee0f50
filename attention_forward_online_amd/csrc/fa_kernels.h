// fa_kernels.h -- host-side launch interface between the C ABI layer and the
// gfx950 kernels.  Arguments reaching these functions have already been
// validated by fa_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
    const void *Q, *K, *V;
    void *O;
    float *LSE;
    const int32_t *key_lens;    // device int32[B] or nullptr
    int B, H, N, Nk, d;
    float scale;                // > 0, finite
    int causal;                 // 0 or 1
};

struct DecodeArgs {
    const void *Q, *K, *V;
    void *O;
    float *LSE;
    const int32_t *key_lens;
    int B, H, Nk, d;
    float scale;
    int num_splits;
    float *workspace;           // B*H*num_splits*(d+2) floats
};

struct SoftmaxArgs {
    const void *X;
    void *Y;                    // nullptr: log-sum-exp only
    float *LSE;
    long long rows, cols;
    void *workspace;            // softmax_workspace_bytes(rows, cols, ...) bytes
};

struct BwdArgs {
    const void *Q, *K, *V, *O, *dO;
    const float *LSE;
    void *dQ, *dK, *dV;
    const int32_t *key_lens;
    int B, H, N, Nk, d;
    float scale;
    int causal;
    void *workspace;            // backward_workspace_bytes(B, H, N) bytes
};

// bf16 prefill, d in {64, 128}: MFMA 32x32x16 bf16 tiles.
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream);

// compute units of the current device (looked up once per device)
int device_cu_count();

// fp32 prefill, 1 <= d <= 256: fp32 FMA tiles.
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);
// split-KV decode: bf16 with d in {64, 128}, fp32 with 1 <= d <= 256; is_bf16
// selects the element type.
hipError_t launch_decode(const DecodeArgs &a, bool is_bf16, hipStream_t stream);
// The decode's fixed per-GPU scratch (used in place of a caller workspace):
// its size, and its device address on the current GPU.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void **ptr);

// Row softmax / log-sum-exp of a [rows, cols] fp32 or bf16 matrix.
size_t softmax_workspace_bytes(long long rows, long long cols, bool is_bf16);
hipError_t launch_softmax(const SoftmaxArgs &a, bool is_bf16, hipStream_t stream);
// FlashAttention V1 loop order (ablation), bf16, d in {64, 128}; the workspace
// holds fp32 O, m, l: forward_v1_workspace_bytes(B, H, N, d) bytes.
size_t forward_v1_workspace_bytes(long long B, long long H, long long N, long long d);
hipError_t launch_fwd_v1(const FwdArgs &a, void *workspace, hipStream_t stream);
// bf16 backward, d in {64, 128}: dQ, dK, dV from Q, K, V, O, dO and the forward's LSE.
size_t backward_workspace_bytes(long long B, long long H, long long N);
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream);
// fp32 backward, 1 <= d <= 256 (same workspace layout).
hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t stream);
// Test hook: polls of the one-pass wait before its fallback (< 0: default).
void set_softmax_spin_limit(int limit);
// Rescale rule of the bf16 prefill: the overflow guard (default), the FA-4
// threshold or the eager per-tile rescale.  Test and ablation hook.
constexpr int kRuleEager = 0, kRuleTau = 1, kRuleGuard = 2;
void set_rescale_rule(int rule);
int rescale_rule();

// measurement probes (fa_probe.hip): a bf16 MFMA stream, a streaming read and
// a streaming copy
hipError_t launch_probe_mfma(float *sink, int blocks, int iters, hipStream_t stream);
hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, int blocks, hipStream_t stream);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, int blocks, hipStream_t stream);

}  // namespace fa
