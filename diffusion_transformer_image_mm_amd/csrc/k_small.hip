// Small kernels around the block: the vector-matrix products of the
// modulation and embedder layers, the sinusoidal timestep embedding, the
// Euler update, the RoPE table and a plain copy.
#include "common.h"

namespace mmdit {

// ---------------------------------------------------------------------------
// out[n] (+)= sum_k W[n,k] act(x[k]) + b[n]
//
// The modulation layers read a [6H, H] weight for one conditioning vector:
// pure weight streaming (HBM-bound, 2 B per weight in bf16/fp16, 1 B in int8).
// act(x) is staged once per workgroup in LDS; each wavefront owns one output
// row at a time and reads it with 16-byte loads, then reduces across lanes.
// ---------------------------------------------------------------------------
template <int WT>
__global__ __launch_bounds__(256) void gemv_kernel(const float* __restrict__ x, int k,
                                                   const void* __restrict__ w,
                                                   const float* __restrict__ scale,
                                                   const uint16_t* __restrict__ bias, int n,
                                                   int silu_input, int accumulate,
                                                   float* __restrict__ out) {
    extern __shared__ float xs[];
    for (int i = threadIdx.x; i < k; i += 256) {
        float v = x[i];
        xs[i] = silu_input ? silu(v) : v;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    constexpr bool INT8 = WT == MMDIT_INT8;
    constexpr int EPL = INT8 ? 16 : 8;  // elements per 16-byte load
    for (int row = wave; row < n; row += nwaves) {
        float acc = 0.f;
        if (INT8) {
            const int8_t* wr = static_cast<const int8_t*>(w) + (size_t)row * k;
            for (int c = lane * EPL; c < k; c += 64 * EPL) {
                const int4 raw = *reinterpret_cast<const int4*>(wr + c);
                const int8_t* e = reinterpret_cast<const int8_t*>(&raw);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc += (float)e[i] * xs[c + i];
            }
        } else {
            const uint16_t* wr = static_cast<const uint16_t*>(w) + (size_t)row * k;
            for (int c = lane * EPL; c < k; c += 64 * EPL) {
                const uint4 raw = *reinterpret_cast<const uint4*>(wr + c);
                const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc += (WT == MMDIT_F16 ? h2f(e[i]) : bf2f(e[i])) * xs[c + i];
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            float y = (INT8 ? acc * scale[row] : acc) + bf2f(bias[row]);
            out[row] = accumulate ? out[row] + y : y;
        }
    }
}

hipError_t launch_gemv(const float* x, int k, const void* w, const float* scale,
                       const uint16_t* bias, int n, int wtype, int silu_input, int accumulate,
                       float* out, hipStream_t s) {
    int blocks = (n + 3) / 4;
    if (blocks > 2048) blocks = 2048;
    const size_t lds = (size_t)k * sizeof(float);
#define GEMV_CASE(T)                                                                               \
    case T:                                                                                        \
        hipLaunchKernelGGL(gemv_kernel<T>, dim3(blocks), dim3(256), lds, s, x, k, w, scale, bias, n, \
                           silu_input, accumulate, out);                                           \
        break;
    switch (wtype) {
        GEMV_CASE(MMDIT_BF16) GEMV_CASE(MMDIT_INT8) GEMV_CASE(MMDIT_F16)
        default: return hipErrorInvalidValue;
    }
#undef GEMV_CASE
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 -> fp16, round to nearest even (the conversion the GEMM applies to
// bf16 weight fragments), 8 values per 16-byte load and store.
// ---------------------------------------------------------------------------
__global__ void bf16_to_f16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                   size_t count) {
    const size_t n8 = count / 8;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
        const uint4 v = reinterpret_cast<const uint4*>(src)[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack2h(__uint_as_float(w[j] << 16), __uint_as_float(w[j] & 0xffff0000u));
        reinterpret_cast<uint4*>(dst)[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    for (size_t i = n8 * 8 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        dst[i] = f2h(bf2f(src[i]));
}

hipError_t launch_bf16_to_f16(const uint16_t* src, uint16_t* dst, size_t count, hipStream_t s) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count / 8 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, count);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sinusoidal embedding of the scalars t and guidance (256 values each):
// [cos(1000 t f_k) | sin(1000 t f_k)], f_k = exp(-ln(1e4) k / 128).
// out[0:256] = emb(t), out[256:512] = emb(guidance). Angles in fp64.
// ---------------------------------------------------------------------------
__global__ void timestep_embedding_kernel(float t, float g, float* __restrict__ out) {
    const int i = threadIdx.x;  // 0..255
    const int k = i & 127;
    const double f = exp(-log(10000.0) * (double)k / 128.0);
    const double at = 1000.0 * (double)t * f, ag = 1000.0 * (double)g * f;
    out[i] = (float)(i < 128 ? cos(at) : sin(at));
    out[256 + i] = (float)(i < 128 ? cos(ag) : sin(ag));
}

hipError_t launch_time_and_guidance_embedding(float t, float g, float* out, hipStream_t s) {
    hipLaunchKernelGGL(timestep_embedding_kernel, dim3(1), dim3(256), 0, s, t, g, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Euler update z += dt v (fp32)
// ---------------------------------------------------------------------------
__global__ void euler_kernel(float* __restrict__ z, const float* __restrict__ v, int64_t n, float dt) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        z[i] += dt * v[i];
}

hipError_t launch_euler(float* z, const float* v, int64_t n, float dt, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(euler_kernel, dim3((unsigned)blocks), dim3(256), 0, s, z, v, n, dt);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RoPE table [L, D/2, 2] (cos, sin) from axial ids [L, 3]; angle in fp64.
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(const int32_t* __restrict__ ids, int seq_len, int half, int a0,
                                  int a1, int a2, double log_theta, float* __restrict__ rope) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)seq_len * half) return;
    const int l = (int)(i / half), p = (int)(i % half);
    int axis, j, da;
    if (p < a0 / 2) { axis = 0; j = p; da = a0; }
    else if (p < (a0 + a1) / 2) { axis = 1; j = p - a0 / 2; da = a1; }
    else { axis = 2; j = p - (a0 + a1) / 2; da = a2; }
    const double freq = exp(-2.0 * (double)j / (double)da * log_theta);
    const double ang = (double)ids[l * 3 + axis] * freq;
    rope[2 * i] = (float)cos(ang);
    rope[2 * i + 1] = (float)sin(ang);
}

hipError_t launch_rope_table(const int32_t* ids, int seq_len, int head_dim, int a0, int a1, int a2,
                             float theta, float* rope, hipStream_t s) {
    const int half = head_dim / 2;
    const int64_t n = (int64_t)seq_len * half;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids,
                       seq_len, half, a0, a1, a2, log((double)theta), rope);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void copy_f32_kernel(float* __restrict__ dst, const float* __restrict__ src, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        reinterpret_cast<float4*>(dst)[i] = reinterpret_cast<const float4*>(src)[i];
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t n4 = n / 4;  // callers pass multiples of 4 (rows of H floats)
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n4);
    return hipGetLastError();
}

}  // namespace mmdit
