// prefill_f32.hip -- attention forward for fp32 inputs (d_h in {16,32,64,128}).
//
// Same method as the bf16 kernel -- K/V tiles staged on chip, a running
// max / sum / unnormalised output per query row, one division at the end
// ("Attention Engineering: From MHA to GQA, MLA & FlashAttention", section 4,
// the FlashAttention-2 recurrence) -- but with fp32 FMAs throughout so that
// fp32 inputs keep fp32 accuracy.  A workgroup covers 64 rows of one query
// head and reads the K/V head h / (h_q / h_kv).  For d_h <= 32 each row's
// keys are split over NSPLIT waves (8 for d_h = 16, 4 for d_h = 32; wave w
// takes keys w, w + NSPLIT, ... of every tile), each with its own running
// (m, l, O); at the end the states of a row merge through LDS as the
// FlashAttention-2 state merge prescribes
// (the same section: rescale each by 2^(m_w - M), add).  For larger heads
// one wave owns the row.  Each dot product runs as four interleaved FMA
// chains.  This path serves small fp32 problems, where the time is latency:
// a tile holds up to 128 keys (16 KB per operand), so the tiny workloads
// load K and V once.
#include "kcommon.h"
#include "kernels.h"

namespace mi355 {
namespace {

constexpr int ROWS = 64;

struct Params {
    const float *q, *k, *v;
    float *o;
    float *lse;
    int T, hq, hkv, G;
    int causal, window;
    float scale_log2;
    const float *sinks;   // [hq] sink logits (natural units) or nullptr
};

template <int DH> struct Shape {
    static constexpr int NSPLIT = DH == 16 ? 8 : (DH == 32 ? 4 : 1);   // waves sharing a row's keys
    static constexpr int TK = DH == 16 ? 128 : (DH == 32 ? 64 : 32);   // keys per LDS tile
};

template <int DH>
__global__ __launch_bounds__(ROWS * Shape<DH>::NSPLIT) void prefill_f32_kernel(Params p) {
    constexpr int NSPLIT = Shape<DH>::NSPLIT;
    constexpr int TK = Shape<DH>::TK;
    constexpr int NT = ROWS * NSPLIT;
    __shared__ float ks[TK][DH];
    __shared__ float vs[TK][DH];
    // per-wave row states for the merge (unused when NSPLIT == 1)
    __shared__ float part_o[NSPLIT > 1 ? NSPLIT : 1][NSPLIT > 1 ? ROWS : 1][DH + 1];
    __shared__ float part_ml[NSPLIT > 1 ? NSPLIT : 1][NSPLIT > 1 ? ROWS : 1][2];
    const int tid = threadIdx.x;
    const int wave = tid / ROWS;
    const int row = blockIdx.x * ROWS + tid % ROWS;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / p.G;
    const int T = p.T;
    const size_t q_base = ((size_t)b * p.hq + h) * (size_t)T * DH;
    const size_t kv_base = ((size_t)b * p.hkv + g) * (size_t)T * DH;

    float q[DH], o[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) {
        q[d] = row < T ? p.q[q_base + (size_t)row * DH + d] : 0.f;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    const int r0 = blockIdx.x * ROWS;
    const int kend = p.causal ? min(T, r0 + ROWS) : T;
    const int kbeg = p.window > 0 ? max(0, r0 - p.window + 1) : 0;
    for (int ts = (kbeg / TK) * TK; ts < kend; ts += TK) {
        for (int c = tid; c < TK * DH; c += NT) {
            const int j = c / DH, d = c % DH;
            const int key = ts + j;
            ks[j][d] = key < T ? p.k[kv_base + (size_t)key * DH + d] : 0.f;
            vs[j][d] = key < T ? p.v[kv_base + (size_t)key * DH + d] : 0.f;
        }
        __syncthreads();
        if (row < T) {
            for (int j = wave; j < TK; j += NSPLIT) {
                const int key = ts + j;
                bool vis = key < T;
                if (p.causal) vis = vis && key <= row;
                if (p.window > 0) vis = vis && (row - key) < p.window;
                if (!vis) continue;
                float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < DH; ++d) sp[d & 3] = fmaf(q[d], ks[j][d], sp[d & 3]);
                const float s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
                const float x = s * p.scale_log2;
                if (x > m) {
                    const float alpha = fast_exp2(m - x);
                    l *= alpha;
#pragma unroll
                    for (int d = 0; d < DH; ++d) o[d] *= alpha;
                    m = x;
                }
                const float pw = fast_exp2(x - m);
                l += pw;
#pragma unroll
                for (int d = 0; d < DH; ++d) o[d] = fmaf(pw, vs[j][d], o[d]);
            }
        }
        __syncthreads();
    }
    if constexpr (NSPLIT > 1) {
        // merge the row's NSPLIT states: M = max m_w, O = sum 2^(m_w - M) O_w,
        // l = sum 2^(m_w - M) l_w (a state with m_w = -inf saw no key)
        const int r = tid % ROWS;
        part_ml[wave][r][0] = m;
        part_ml[wave][r][1] = l;
#pragma unroll
        for (int d = 0; d < DH; ++d) part_o[wave][r][d] = o[d];
        __syncthreads();
        if (wave != 0) return;
        float mw[NSPLIT];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NSPLIT; ++w) {
            mw[w] = part_ml[w][r][0];
            M = fmaxf(M, mw[w]);
        }
        l = 0.f;
#pragma unroll
        for (int d = 0; d < DH; ++d) o[d] = 0.f;
#pragma unroll
        for (int w = 0; w < NSPLIT; ++w) {
            const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
            l = fmaf(f, part_ml[w][r][1], l);
#pragma unroll
            for (int d = 0; d < DH; ++d) o[d] = fmaf(f, part_o[w][r][d], o[d]);
        }
        m = M;
    }
    if (row >= T) return;
    float inv = l > 0.f ? 1.0f / l : 0.f;
    float lse_out = l > 0.f ? m * kLn2 + __logf(l) : -INFINITY;
    if (p.sinks) inv = finish_row_with_sink(m, l, p.sinks[h] * kLog2e, lse_out);
#pragma unroll
    for (int d = 0; d < DH; ++d) p.o[q_base + (size_t)row * DH + d] = o[d] * inv;
    if (p.lse) p.lse[((size_t)b * p.hq + h) * (size_t)T + row] = lse_out;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const float *>(a.q);
    p.k = static_cast<const float *>(a.k);
    p.v = static_cast<const float *>(a.v);
    p.o = static_cast<float *>(a.o);
    p.lse = a.lse;
    p.T = a.T;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.G = a.hq / a.hkv;
    p.causal = a.causal;
    p.window = a.window;
    p.scale_log2 = a.scale * kLog2e;
    p.sinks = a.sinks;
    dim3 grid((a.T + ROWS - 1) / ROWS, a.hq, a.B);
    switch (a.d) {
        case 16: hipLaunchKernelGGL(prefill_f32_kernel<16>, grid, dim3(ROWS * Shape<16>::NSPLIT), 0, stream, p); break;
        case 32: hipLaunchKernelGGL(prefill_f32_kernel<32>, grid, dim3(ROWS * Shape<32>::NSPLIT), 0, stream, p); break;
        case 64: hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(ROWS * Shape<64>::NSPLIT), 0, stream, p); break;
        case 128: hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(ROWS * Shape<128>::NSPLIT), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mi355
