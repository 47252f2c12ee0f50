// fa_fwd_f32.hip -- fp32 prefill attention forward (any 1 <= d <= 256).
//
// The same tile recurrence as the bf16 path ('Online Softmax -- the
// mathematical heart of FlashAttention', sections 4-5), with every product and
// sum in fp32 on the vector ALUs: no reduced-precision matrix instruction
// touches the data.  LPR lanes share a query row and split its d dimension in
// 4-float pieces, so a score is LPR partial dot products combined by lane
// exchanges (DPP) inside the row's lane group; a workgroup of 256 threads holds
// 256 / LPR rows.  LPR = 4 in general; small grids take LPR = 16, which gives
// four times the waves and a quarter of the per-lane work per key, and the
// smallest (fewer 16-row blocks than CUs, e.g. one 256-row head) also split
// each block's keys over its four waves (4 rows per workgroup, key tiles
// dealt round-robin to the waves, states merged at the end), which shortens
// the serial key loop of every row four times.  K/V tiles of 32 keys are staged in LDS,
// zero-padded to the compiled width DMAX (zeros add nothing to a dot product
// and the padded output columns are never stored).
// Fully masked rows give O = 0 and LSE = -inf as in the bf16 path.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBc = 32;               // keys per tile

// sum over the LPR lanes of a row group (LPR = 4: quad; 16: DPP row)
template <int LPR>
__device__ __forceinline__ float row_group_sum(float x) {
    if constexpr (LPR == 16) {
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));   // row_ror:8
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));   // row_ror:4
    }
    x += quad_xor_f32<1>(x);
    x += quad_xor_f32<2>(x);
    return x;
}

// KW > 1 (small grids): the workgroup's threads form KW "ways" of kThreads / KW
// lanes over the same rows; way w takes the key tiles w, w + KW, w + 2 KW, ...
// with its own LDS tile, and the ways' states are merged at the end.
template <int DMAX, int LPR, int KW>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ key_lens,
    int H, int N, int Nk, int d, int causal, int n_qtiles, float c) {
    constexpr int TW = kThreads / KW;       // threads per way
    constexpr int kRows = TW / LPR;         // query rows per workgroup
    constexpr int NCH = DMAX / (4 * LPR);   // 4-float pieces per lane
    static_assert(NCH >= 1 && NCH * 4 * LPR == DMAX, "width/lane split");
    static_assert(KW == 1 || TW % 64 == 0, "a way is whole waves");
    __shared__ __attribute__((aligned(16))) float Ks[KW * kBc * DMAX];
    __shared__ __attribute__((aligned(16))) float Vs[KW * kBc * DMAX];

    const int tid = threadIdx.x, way = tid / TW, wtid = tid % TW, part = wtid % LPR;
    const int qtile = blockIdx.x % n_qtiles, bh = blockIdx.x / n_qtiles, b = bh / H;
    const int qrow = qtile * kRows + wtid / LPR;
    float *const Kw = Ks + way * (kBc * DMAX);
    float *const Vw = Vs + way * (kBc * DMAX);
    const int off = Nk - N;
    const int kv_lim = visible_len(key_lens, b, Nk);
    int kv_end = kv_lim;
    if (causal) kv_end = min(kv_end, min(qtile * kRows + kRows, N) - 1 + off + 1);
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
    const size_t q_base = (size_t)bh * N * d, kv_base = (size_t)bh * Nk * d;

    float q[NCH][4], o[NCH][4];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 4 * LPR * k + 4 * part + e;
            q[k][e] = (qrow < N && col < d) ? Q[q_base + (size_t)qrow * d + col] : 0.f;
            o[k][e] = 0.f;
        }
    // the running denominator is l + lc: each tile's sum of weights is added
    // with an error-free two-sum whose rounding error accumulates in lc, so a
    // row over millions of keys keeps fp32 accuracy in LSE
    float ms = neg_inf(), l = 0.f, lc = 0.f;

    // K/V tiles: all of a thread's loads are issued at once, and (up to
    // DMAX = 64, where the registers allow it without losing a wave) the next
    // tile's loads are in flight while the current one is computed
    constexpr bool kPrefetch = DMAX <= 64;
    const rsrc_t ksrc = make_rsrc(K + kv_base, (uint32_t)max(kv_end, 0) * d * 4);
    const rsrc_t vsrc = make_rsrc(V + kv_base, (uint32_t)max(kv_end, 0) * d * 4);
    F32TileStage<kBc, DMAX, TW> kst, vst;
    if (kPrefetch && way < ntiles) {
        kst.load(ksrc, way * kBc, d, wtid);
        vst.load(vsrc, way * kBc, d, wtid);
    }
    // every way runs the same number of iterations (one barrier pair each);
    // a way past its last tile only joins the barriers
    const int nit = (ntiles + KW - 1) / KW;
    for (int it = 0; it < nit; ++it) {
        const int t = it * KW + way;
        const int j0 = t * kBc;
        if (!kPrefetch && t < ntiles) {
            kst.load(ksrc, j0, d, wtid);
            vst.load(vsrc, j0, d, wtid);
        }
        __syncthreads();   // previous tile fully consumed
        if (t < ntiles) {
            kst.store(Kw, wtid);
            vst.store(Vw, wtid);
        }
        __syncthreads();
        if (t >= ntiles) continue;
        if (kPrefetch && t + KW < ntiles) {
            kst.load(ksrc, j0 + KW * kBc, d, wtid);
            vst.load(vsrc, j0 + KW * kBc, d, wtid);
        }

        // keys are taken in groups whose K rows are read from LDS in one batch
        // (16 16-byte reads), so a wave waits once per group, not per key
        constexpr int KG = NCH >= 16 ? 1 : 16 / NCH;
        float s[kBc];
#pragma unroll
        for (int jg = 0; jg < kBc; jg += KG) {
            f32x4_t kv[KG][NCH];
#pragma unroll
            for (int u = 0; u < KG; ++u)
#pragma unroll
                for (int k = 0; k < NCH; ++k) kv[u][k] = *(const f32x4_t *)&Kw[(jg + u) * DMAX + 4 * LPR * k + 4 * part];
#pragma unroll
            for (int u = 0; u < KG; ++u) {
                float part_dot = 0.f;
#pragma unroll
                for (int k = 0; k < NCH; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) part_dot = fmaf(q[k][e], kv[u][k][e], part_dot);
                part_dot = row_group_sum<LPR>(part_dot);
                const int key = j0 + jg + u;
                const bool ok = key < kv_lim && (!causal || key <= qrow + off);
                s[jg + u] = ok ? part_dot : neg_inf();
            }
        }
        float mx = s[0];
#pragma unroll
        for (int jj = 1; jj < kBc; ++jj) mx = fmaxf(mx, s[jj]);
        const float ms_new = fmaxf(ms, mx * c);
        const float ms_ref = ms_new == neg_inf() ? 0.f : ms_new;   // -inf guard
        const float alpha = exp2_hw(ms - ms_ref);
        ms = ms_new;
        l *= alpha;
        lc *= alpha;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[k][e] *= alpha;
        float lt = 0.f;   // this tile's weights
#pragma unroll
        for (int jg = 0; jg < kBc; jg += KG) {
            f32x4_t vv[KG][NCH];
#pragma unroll
            for (int u = 0; u < KG; ++u)
#pragma unroll
                for (int k = 0; k < NCH; ++k) vv[u][k] = *(const f32x4_t *)&Vw[(jg + u) * DMAX + 4 * LPR * k + 4 * part];
#pragma unroll
            for (int u = 0; u < KG; ++u) {
                const float p = exp2_hw(fmaf(s[jg + u], c, -ms_ref));
                lt += p;
#pragma unroll
                for (int k = 0; k < NCH; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[k][e] = fmaf(p, vv[u][k][e], o[k][e]);
            }
        }
        const float ls = l + lt, bv = ls - l;
        lc += (l - (ls - bv)) + (lt - bv);
        l = ls;
    }
    l += lc;

    if constexpr (KW > 1) {
        // ways 1.. hand (ms, l, o) to way 0 through LDS (per lane, 2 + 4 NCH
        // floats); way 0 merges them in way order with the (m, l) merge
        // ('Online Softmax & FlashAttention', Step 1)
        constexpr int NV = 2 + 4 * NCH;
        static_assert((KW - 1) * TW * NV <= KW * kBc * DMAX, "merge state does not fit");
        __syncthreads();   // every way is past its last LDS read
        if (way > 0) {
            float *st = Ks + ((way - 1) * NV) * TW + wtid;
            st[0] = ms;
            st[TW] = l;
#pragma unroll
            for (int k = 0; k < NCH; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[(2 + 4 * k + e) * TW] = o[k][e];
        }
        __syncthreads();
        if (way > 0) return;
#pragma unroll
        for (int w = 1; w < KW; ++w) {
            const float *st = Ks + ((w - 1) * NV) * TW + wtid;
            const float ms2 = st[0], l2 = st[TW];
            const float mm = fmaxf(ms, ms2);
            const float a1 = ms == neg_inf() ? 0.f : exp2_hw(ms - mm);
            const float a2 = ms2 == neg_inf() ? 0.f : exp2_hw(ms2 - mm);
            l = a1 * l + a2 * l2;
#pragma unroll
            for (int k = 0; k < NCH; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[k][e] = a1 * o[k][e] + a2 * st[(2 + 4 * k + e) * TW];
            ms = mm;
        }
    }
    if (qrow < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 4 * LPR * k + 4 * part + e;
                if (col < d) O[q_base + (size_t)qrow * d + col] = o[k][e] * inv;
            }
        if (part == 0)
            LSE[(size_t)bh * N + qrow] = l > 0.f ? (ms + log2_hw(l)) * kLn2 : neg_inf();
    }
}

template <int DMAX, int LPR, int KW = 1>
hipError_t launch_one(const FwdArgs &a, hipStream_t stream) {
    constexpr int kRows = kThreads / KW / LPR;
    const int n_qtiles = (a.N + kRows - 1) / kRows;
    const long long nblocks = (long long)a.B * a.H * n_qtiles;
    hipLaunchKernelGGL((fwd_f32_kernel<DMAX, LPR, KW>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                       (const float *)a.Q, (const float *)a.K, (const float *)a.V, (float *)a.O,
                       a.LSE, a.key_lens, a.H, a.N, a.Nk, a.d, a.causal, n_qtiles,
                       a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream) {
    // fewer 64-row workgroups than CUs (half as many for d > 128): 16 lanes per
    // row instead of 4 (measured: 2-3x on such grids, slower beyond them)
    // fewer 16-row workgroups than that: 4-row workgroups whose four waves
    // split the keys (four times the workgroups, a quarter of the serial key
    // loop per wave)
    const long long blocks4 = (long long)a.B * a.H * ((a.N + 63) / 64);
    const long long blocks16 = (long long)a.B * a.H * ((a.N + 15) / 16);
    if (a.d <= 16) return launch_one<16, 4>(a, stream);
    if (a.d <= 64) {
        if (blocks16 < 256) return launch_one<64, 16, 4>(a, stream);
        return blocks4 < 256 ? launch_one<64, 16>(a, stream) : launch_one<64, 4>(a, stream);
    }
    if (a.d <= 128) {
        if (blocks16 < 256) return launch_one<128, 16, 4>(a, stream);
        return blocks4 < 256 ? launch_one<128, 16>(a, stream) : launch_one<128, 4>(a, stream);
    }
    return blocks4 < 128 ? launch_one<256, 16>(a, stream) : launch_one<256, 4>(a, stream);
}

}  // namespace fa
