// Embedding gather, RMSNorm, RoPE table, argmax and small device-counter kernels.
#include "launch.hpp"

namespace lk {

// cos and sin of pos * theta_i, theta_i = theta^(-i/(d/2)); the angle and both functions in
// double precision, rounded to float (article, section 位置编码).
__global__ void rope_table_kernel(float2* rope, int max_seq, int half, double theta) {
    const int pos = blockIdx.x;
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        const double freq = 1.0 / pow(theta, (double)i / (double)half);
        const double ang = (double)pos * freq;
        rope[(size_t)pos * half + i] = make_float2((float)cos(ang), (float)sin(ang));
    }
}

hipError_t rope_table(float2* rope, int max_seq, int d, float theta, hipStream_t s) {
    rope_table_kernel<<<max_seq, 64, 0, s>>>(rope, max_seq, d / 2, (double)theta);
    return hipGetLastError();
}

// x[r] = E[tokens[r]] widened to fp32 (article, section 分词器与编码).  Ids outside [0,V)
// give a zero row and raise DEVERR_TOKEN_RANGE.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int* tokens, const T* E, float* x,
                                                    int D, int V, uint32_t* err) {
    const int r = blockIdx.x;
    const int tok = tokens[r];
    float* xr = x + (size_t)r * D;
    if (tok < 0 || tok >= V) {
        if (threadIdx.x == 0) atomicOr(err, DEVERR_TOKEN_RANGE);
        for (int i = threadIdx.x; i < D; i += blockDim.x) xr[i] = 0.0f;
        return;
    }
    const T* er = E + (size_t)tok * D;
    for (int i = threadIdx.x * 8; i < D; i += blockDim.x * 8) {
        float v[8];
        load8(er + i, v);
        *reinterpret_cast<f32x4*>(xr + i) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(xr + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

hipError_t embed(Dt dt, const int* tokens, const void* E, float* x, int rows, int D, int V,
                 uint32_t* err, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    if (dt == Dt::BF16)
        embed_kernel<bf16><<<rows, 256, 0, s>>>(tokens, (const bf16*)E, x, D, V, err);
    else
        embed_kernel<float><<<rows, 256, 0, s>>>(tokens, (const float*)E, x, D, V, err);
    return hipGetLastError();
}

// y = x * 1/sqrt(mean(x^2) + eps) * w per row (article, section 分词器与编码; also the
// pitchhut deep-dive's layer-normalisation example).  One block of NT threads per row, each
// thread holding MAXV chunks of 8 values in registers between the two passes (NT * 8 * MAXV
// >= D, D % 8 == 0).
//
// With nsplit > 0 the row first takes the pending split-K sums of the residual GEMM that
// wrote it: x' = x + parts[0] + parts[1] + ... (in that order), stored to x_out.  NSMAX > 0
// handles nsplit <= NSMAX with every load of the row (x and all splits) issued before the
// first add, so a decode-sized launch (few rows) waits for one round trip to memory instead
// of one per chunk; NSMAX < 0 takes any nsplit in groups of four.
template <typename T, int NT, int MAXV, int NSMAX>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(const float* x, int in_step, int in_off,
                                                     const T* w, T* y, int y_pack, int D,
                                                     float eps, const float* parts, int nsplit,
                                                     size_t split_stride, float* x_out) {
    const int r = blockIdx.x;
    const size_t row = ((size_t)r * in_step + in_off) * D;
    const float* xr = x + row;
    float v[MAXV][8];
    float ss = 0.0f;
    // The loads are unconditional (chunks past D re-read the last one and are not used): a
    // branch around a load makes the compiler wait for every load in flight at the join.
    // The weights do not depend on the row: their loads go out first.
    float wv[MAXV][8];
#pragma unroll
    for (int c = 0; c < MAXV; ++c) {
        const int i = (threadIdx.x + c * NT) * 8;
        load8(w + (i < D ? i : D - 8), wv[c]);
    }
    if constexpr (NSMAX >= 0) {
        // indices past the last split re-read it and are not added
        constexpr int NP = NSMAX > 0 ? NSMAX : 1;
        f32x4 xa[MAXV][2], pa[MAXV][NP][2];
#pragma unroll
        for (int c = 0; c < MAXV; ++c) {
            const int i0 = (threadIdx.x + c * NT) * 8, i = i0 < D ? i0 : D - 8;
            xa[c][0] = *reinterpret_cast<const f32x4*>(xr + i);
            xa[c][1] = *reinterpret_cast<const f32x4*>(xr + i + 4);
#pragma unroll
            for (int u = 0; u < NSMAX; ++u) {
                const int z = u < nsplit ? u : nsplit - 1;
                const float* pr = parts + z * split_stride + row + i;
                pa[c][u][0] = *reinterpret_cast<const f32x4*>(pr);
                pa[c][u][1] = *reinterpret_cast<const f32x4*>(pr + 4);
            }
        }
#pragma unroll
        for (int c = 0; c < MAXV; ++c) {
            const int i = (threadIdx.x + c * NT) * 8;
            if (i < D) {
#pragma unroll
                for (int j = 0; j < 4; ++j) { v[c][j] = xa[c][0][j]; v[c][4 + j] = xa[c][1][j]; }
#pragma unroll
                for (int u = 0; u < NSMAX; ++u)
                    if (u < nsplit) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) { v[c][j] += pa[c][u][0][j]; v[c][4 + j] += pa[c][u][1][j]; }
                    }
                if (nsplit > 0) {
                    store4(x_out + row + i, v[c]);
                    store4(x_out + row + i + 4, v[c] + 4);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) ss += v[c][j] * v[c][j];
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < MAXV; ++c) {
            const int i = (threadIdx.x + c * NT) * 8;
            if (i < D) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(xr + i);
                const f32x4 b = *reinterpret_cast<const f32x4*>(xr + i + 4);
                v[c][0] = a[0]; v[c][1] = a[1]; v[c][2] = a[2]; v[c][3] = a[3];
                v[c][4] = b[0]; v[c][5] = b[1]; v[c][6] = b[2]; v[c][7] = b[3];
                // splits in groups of four, each group's loads issued together
                for (int z0 = 0; z0 < nsplit; z0 += 4) {
                    f32x4 pa[4], pb[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int z = z0 + u < nsplit ? z0 + u : nsplit - 1;
                        const float* pr = parts + z * split_stride + row + i;
                        pa[u] = *reinterpret_cast<const f32x4*>(pr);
                        pb[u] = *reinterpret_cast<const f32x4*>(pr + 4);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (z0 + u < nsplit) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) { v[c][j] += pa[u][j]; v[c][4 + j] += pb[u][j]; }
                        }
                }
                if (nsplit > 0) {
                    store4(x_out + row + i, v[c]);
                    store4(x_out + row + i + 4, v[c] + 4);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) ss += v[c][j] * v[c][j];
            }
        }
    }
    constexpr int NWAVE = NT / 64;
    __shared__ float red[NWAVE];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float total = 0.0f;
#pragma unroll
    for (int k = 0; k < NWAVE; ++k) total += red[k];
    const float inv = 1.0f / sqrtf(total / (float)D + eps);
#pragma unroll
    for (int c = 0; c < MAXV; ++c) {
        const int i = (threadIdx.x + c * NT) * 8;
        if (i < D) {
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = (v[c][j] * inv) * wv[c][j];
            T* yr = y + act_offset(r, i, D, y_pack);  // 8 consecutive values stay contiguous
            store4(yr, o);
            store4(yr + 4, o + 4);
        }
    }
}

template <typename T, int NT, int MAXV>
static void rmsnorm_launch(const float* x, int step, int off, const T* w, T* y, int y_pack,
                           int rows, int D, float eps, const float* parts, int nsplit,
                           size_t split_stride, float* x_out, hipStream_t s) {
    if (nsplit == 0)
        rmsnorm_kernel<T, NT, MAXV, 0><<<rows, NT, 0, s>>>(x, step, off, w, y, y_pack, D, eps,
                                                          parts, nsplit, split_stride, x_out);
    else if (nsplit <= 4)
        rmsnorm_kernel<T, NT, MAXV, 4><<<rows, NT, 0, s>>>(x, step, off, w, y, y_pack, D, eps,
                                                          parts, nsplit, split_stride, x_out);
    else
        rmsnorm_kernel<T, NT, MAXV, -1><<<rows, NT, 0, s>>>(x, step, off, w, y, y_pack, D, eps,
                                                           parts, nsplit, split_stride, x_out);
}

// one 8-value chunk per thread up to D = 8192, then two (D <= 16384, the largest dim taken)
template <typename T>
static hipError_t rmsnorm_t(const float* x, int step, int off, const T* w, T* y, int y_pack,
                            int rows, int D, float eps, const float* parts, int nsplit,
                            size_t split_stride, float* x_out, hipStream_t s) {
    if (D <= 2048)
        rmsnorm_launch<T, 256, 1>(x, step, off, w, y, y_pack, rows, D, eps, parts, nsplit, split_stride, x_out, s);
    else if (D <= 4096)
        rmsnorm_launch<T, 512, 1>(x, step, off, w, y, y_pack, rows, D, eps, parts, nsplit, split_stride, x_out, s);
    else if (D <= 8192)
        rmsnorm_launch<T, 1024, 1>(x, step, off, w, y, y_pack, rows, D, eps, parts, nsplit, split_stride, x_out, s);
    else
        rmsnorm_launch<T, 1024, 2>(x, step, off, w, y, y_pack, rows, D, eps, parts, nsplit, split_stride, x_out, s);
    return hipGetLastError();
}

hipError_t rmsnorm_fold(Dt dt, const float* x, const float* parts, int nsplit, size_t split_stride,
                        float* x_out, int in_row_step, int in_row_offset, const void* w, void* y,
                        int y_pack, int rows, int D, float eps, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    if (nsplit < 0 || (nsplit > 0 && (!parts || !x_out))) return hipErrorInvalidValue;
    if (dt == Dt::BF16)
        return rmsnorm_t<bf16>(x, in_row_step, in_row_offset, (const bf16*)w, (bf16*)y, y_pack, rows,
                               D, eps, parts, nsplit, split_stride, x_out, s);
    return rmsnorm_t<float>(x, in_row_step, in_row_offset, (const float*)w, (float*)y, y_pack, rows,
                            D, eps, parts, nsplit, split_stride, x_out, s);
}

hipError_t rmsnorm(Dt dt, const float* x, int in_row_step, int in_row_offset, const void* w,
                   void* y, int y_pack, int rows, int D, float eps, hipStream_t s) {
    return rmsnorm_fold(dt, x, nullptr, 0, 0, nullptr, in_row_step, in_row_offset, w, y, y_pack,
                        rows, D, eps, s);
}

// Greedy choice per row: the largest logit, lowest index among equals (article, section
// 预测下一个输出, torch.argmax).  NaN raises DEVERR_NAN_LOGIT.  Two stages: blocks of
// ARGMAX_CHUNK logits each write their (max, index), then one wave per row reduces them and
// writes out[r] and, if out2 is set, out2[(*counter) * out2_step + r] (the token log of a
// decode loop).
constexpr int ARGMAX_CHUNK = 4096;

__device__ __forceinline__ void better(float& best, int& idx, float v, int i) {
    if (v > best || (v == best && i < idx)) { best = v; idx = i; }
}

__global__ __launch_bounds__(256) void argmax_partial_kernel(const float* logits, int V,
                                                             int row_step, int row_off,
                                                             float* pv, int* pi, int nchunks,
                                                             uint32_t* err) {
    const int c = blockIdx.x, r = blockIdx.y;
    const float* lr = logits + ((size_t)r * row_step + row_off) * V;
    const int lo = c * ARGMAX_CHUNK, hi = min(V, lo + ARGMAX_CHUNK);
    float best = -INFINITY;
    int idx = 0x7fffffff;
    bool nan = false;
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
        const float v = lr[i];
        nan |= (v != v);
        better(best, idx, v, i);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, WAVE);
        const int oi = __shfl_xor(idx, o, WAVE);
        better(best, idx, ob, oi);
    }
    __shared__ float sb[4];
    __shared__ int si[4];
    if (nan) atomicOr(err, DEVERR_NAN_LOGIT);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sb[w] = best; si[w] = idx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        best = sb[0]; idx = si[0];
        for (int k = 1; k < 4; ++k) better(best, idx, sb[k], si[k]);
        pv[(size_t)r * nchunks + c] = best;
        pi[(size_t)r * nchunks + c] = idx;
    }
}

__global__ __launch_bounds__(64) void argmax_final_kernel(const float* pv, const int* pi,
                                                          int nchunks, int* out, int* out2,
                                                          int out2_step, const int* counter) {
    const int r = blockIdx.x;
    float best = -INFINITY;
    int idx = 0x7fffffff;
    for (int c = threadIdx.x; c < nchunks; c += 64)
        better(best, idx, pv[(size_t)r * nchunks + c], pi[(size_t)r * nchunks + c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, WAVE);
        const int oi = __shfl_xor(idx, o, WAVE);
        better(best, idx, ob, oi);
    }
    if (threadIdx.x == 0) {
        if (idx == 0x7fffffff) idx = 0;  // all -inf or NaN
        out[r] = idx;
        if (out2) out2[(size_t)(*counter) * out2_step + r] = idx;
    }
}

size_t argmax_scratch_bytes(int rows, int V) {
    const size_t nchunks = (V + ARGMAX_CHUNK - 1) / ARGMAX_CHUNK;
    return (size_t)rows * nchunks * 8;
}

hipError_t argmax(const float* logits, int rows, int row_step, int row_off, int V, int* out,
                  int* out2, int out2_step, const int* counter, void* scratch, uint32_t* err,
                  hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int nchunks = (V + ARGMAX_CHUNK - 1) / ARGMAX_CHUNK;
    float* pv = static_cast<float*>(scratch);
    int* pi = reinterpret_cast<int*>(pv + (size_t)rows * nchunks);
    argmax_partial_kernel<<<dim3(nchunks, rows), 256, 0, s>>>(logits, V, row_step, row_off, pv,
                                                              pi, nchunks, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    argmax_final_kernel<<<rows, 64, 0, s>>>(pv, pi, nchunks, out, out2, out2_step, counter);
    return hipGetLastError();
}

__global__ void bump_counters_kernel(int* pos, int* step) {
    if (threadIdx.x == 0) { *pos += 1; *step += 1; }
}
hipError_t bump_counters(int* pos, int* step, hipStream_t s) {
    bump_counters_kernel<<<1, 64, 0, s>>>(pos, step);
    return hipGetLastError();
}

__global__ void set_counters_kernel(int* pos, int pos_value, int* step) {
    if (threadIdx.x == 0) { *pos = pos_value; *step = 0; }
}
hipError_t set_counters(int* pos, int pos_value, int* step, hipStream_t s) {
    set_counters_kernel<<<1, 64, 0, s>>>(pos, pos_value, step);
    return hipGetLastError();
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}
hipError_t zero_u32(uint32_t* p, int n, hipStream_t s) {
    zero_u32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n);
    return hipGetLastError();
}

__global__ void zero_bytes_kernel(u32x4* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}
hipError_t zero_bytes(void* p, size_t bytes, hipStream_t s) {
    if (bytes % 16 != 0 || ((uintptr_t)p % 16) != 0) return hipErrorInvalidValue;
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    const size_t want = (n + 255) / 256;
    zero_bytes_kernel<<<(unsigned)(want < 8192 ? want : 8192), 256, 0, s>>>((u32x4*)p, n);
    return hipGetLastError();
}

__global__ void check_positions_kernel(const int* pos, int B, int max_pos, uint32_t* err) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B && (pos[b] < 0 || pos[b] >= max_pos)) atomicOr(err, DEVERR_POSITION_RANGE);
}
hipError_t check_positions(const int* pos, int B, int max_pos, uint32_t* err, hipStream_t s) {
    check_positions_kernel<<<(B + 255) / 256, 256, 0, s>>>(pos, B, max_pos, err);
    return hipGetLastError();
}

// dst[r][0..D) = src[r * step + off][0..D) for r < rows (fp32 rows, D % 4 == 0)
__global__ __launch_bounds__(256) void copy_rows_kernel(const float* src, int step, int off,
                                                        float* dst, int D) {
    const size_t r = blockIdx.x;
    const f32x4* in = reinterpret_cast<const f32x4*>(src + (r * step + off) * D);
    f32x4* out = reinterpret_cast<f32x4*>(dst + r * D);
    for (int i = threadIdx.x; i < D / 4; i += blockDim.x) out[i] = in[i];
}
hipError_t copy_rows(const float* src, int step, int off, float* dst, int rows, int D,
                     hipStream_t s) {
    if (rows == 0) return hipSuccess;
    copy_rows_kernel<<<rows, 256, 0, s>>>(src, step, off, dst, D);
    return hipGetLastError();
}

__global__ void copy_tokens_kernel(const int* src, int* dst, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}
hipError_t copy_tokens(const int* src, int* dst, int n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    copy_tokens_kernel<<<(n + 255) / 256, 256, 0, s>>>(src, dst, n);
    return hipGetLastError();
}

}  // namespace lk
