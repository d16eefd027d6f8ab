// Causal grouped-query attention over the KV cache (article, sections 查询和键相乘, 掩码,
// 注意力向量, 多头注意力): for query head h of the token at position p,
//   o = sum_{n <= p} softmax_n(q . k_n / sqrt(d)) v_n,  k and v of KV head h / (H/G).
// Cache layout: K [b][g][pos][d] (seq_stride positions per (b, g)), V transposed
// [b][g][d][pos].
#include "launch.hpp"

namespace lk {

namespace {

// Generic path (any even d <= 256, fp32 or bf16): one wave per (query row, head), keys in
// chunks of 64 (one per lane) with an online softmax; lane owns output dims lane + 64 i.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ kc,
                                                           const T* __restrict__ vc,
                                                           T* __restrict__ out, int S,
                                                           int start_pos, const int* pos_dev,
                                                           int H, int G, int d, int seq_stride,
                                                           float scale_log2) {
    const int row = blockIdx.x;  // b * S + s
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int b = row / S, s = row - b * S;
    const int qpos = (pos_dev ? *pos_dev : start_pos) + s;
    const int g = h / (H / G);
    __shared__ float qs[256];
    const T* qr = q + (size_t)row * H * d + (size_t)h * d;
    for (int i = lane; i < d; i += 64) qs[i] = to_f32(qr[i]);
    __syncthreads();

    const T* kb = kc + ((size_t)b * G + g) * seq_stride * d;
    const T* vb = vc + ((size_t)b * G + g) * d * seq_stride;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    const int nkeys = qpos + 1;
    for (int c0 = 0; c0 < nkeys; c0 += 64) {
        const int j = c0 + lane;
        float sc = -INFINITY;
        if (j < nkeys) {
            const T* kr = kb + (size_t)j * d;
            float acc = 0.f;
            for (int i = 0; i < d; ++i) acc = fmaf(qs[i], to_f32(kr[i]), acc);
            sc = acc * scale_log2;  // score in log2 units
        }
        const float cmax = wave_max(sc);
        const float mnew = fmaxf(mrun, cmax);
        const float corr = exp2f(mrun - mnew);  // 0 on the first chunk (mrun = -inf)
        const float p = (j < nkeys) ? exp2f(sc - mnew) : 0.f;
        lrun = lrun * corr + wave_sum(p);
        mrun = mnew;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= corr;
        const int cn = min(64, nkeys - c0);
        for (int jj = 0; jj < cn; ++jj) {
            const float pj = __shfl(p, jj, 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dd = lane + 64 * i;
                if (dd < d) o[i] = fmaf(pj, to_f32(vb[(size_t)dd * seq_stride + c0 + jj]), o[i]);
            }
        }
    }
    T* orow = out + (size_t)row * H * d + (size_t)h * d;
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dd = lane + 64 * i;
        if (dd < d) orow[dd] = from_f32<T>(o[i] * inv);
    }
}

template <typename T>
hipError_t launch_generic(const AttnArgs& a, hipStream_t s) {
    const int rows = a.B * a.S;
    if (rows == 0) return hipSuccess;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)a.d);
    dim3 grid(rows, a.H);
    attn_generic_kernel<T><<<grid, 64, 0, s>>>((const T*)a.q, (const T*)a.kc, (const T*)a.vc,
                                               (T*)a.out, a.S, a.start_pos, a.pos_dev, a.H, a.G,
                                               a.d, a.seq_stride, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t attention_prefill(Dt dt, const AttnArgs& a, hipStream_t s) {
    if (dt == Dt::BF16) return launch_generic<bf16>(a, s);
    return launch_generic<float>(a, s);
}

hipError_t attention_decode(Dt dt, const AttnArgs& a, hipStream_t s) {
    if (dt == Dt::BF16) return launch_generic<bf16>(a, s);
    return launch_generic<float>(a, s);
}

}  // namespace lk
