// LayerNorm + adaLN modulate: fp32 residual rows -> fp16 GEMM operand.
//
// Luminal blog, "What the compiler found on its own": LayerNorm is a mean, a
// subtraction, a square-sum and a reciprocal square root; the adaLN
// modulation after it is a scale and a shift. Here: out = LN(x)(1+scale)+shift
// with a biased variance and no affine.
//
// The output is the activation operand of the next projection, stored as
// fp16 (10-bit significand; LayerNorm outputs are O(10), far inside fp16's
// range). HBM-bound: each row is read once (4 B/elem), written once (2 B/elem).
// One wavefront owns one row and keeps it in registers (VPT float4 per lane),
// so the two-pass mean/variance costs no second HBM read. 128-bit loads,
// 64-bit stores, butterfly reductions within the wavefront.
#include "common.h"

namespace mmdit {

template <int VPT>
__global__ __launch_bounds__(256) void ln_modulate_kernel(
    const float* __restrict__ x, int rows, int hidden, int split,
    const float* __restrict__ shift0, const float* __restrict__ scale0,
    const float* __restrict__ shift1, const float* __restrict__ scale1, float eps,
    uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * hidden);
    const int n4 = hidden >> 2;
    float4 v[VPT];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        int c = i * 64 + lane;
        if (c < n4) {
            v[i] = xr[c];
            s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        } else {
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const float inv_h = 1.0f / (float)hidden;
    const float mean = wave_sum(s) * inv_h;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        int c = i * 64 + lane;
        if (c < n4) {
            float a = v[i].x - mean, b = v[i].y - mean, cc = v[i].z - mean, d = v[i].w - mean;
            q += (a * a + b * b) + (cc * cc + d * d);
        }
    }
    const float var = wave_sum(q) * inv_h;
    const float rstd = 1.0f / sqrtf(var + eps);
    const bool first = row < split;
    const float4* sh = reinterpret_cast<const float4*>(first ? shift0 : shift1);
    const float4* sc = reinterpret_cast<const float4*>(first ? scale0 : scale1);
    uint2* orow = reinterpret_cast<uint2*>(out + (size_t)row * hidden);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        int c = i * 64 + lane;
        if (c < n4) {
            float4 a = sh[c], b = sc[c];
            float y0 = (v[i].x - mean) * rstd * (1.0f + b.x) + a.x;
            float y1 = (v[i].y - mean) * rstd * (1.0f + b.y) + a.y;
            float y2 = (v[i].z - mean) * rstd * (1.0f + b.z) + a.z;
            float y3 = (v[i].w - mean) * rstd * (1.0f + b.w) + a.w;
            orow[c] = make_uint2(pack2h(y0, y1), pack2h(y2, y3));
        }
    }
}

hipError_t launch_ln_modulate(const float* x, int rows, int hidden, int split,
                              const float* shift0, const float* scale0,
                              const float* shift1, const float* scale1, float eps,
                              uint16_t* out, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    dim3 grid((rows + 3) / 4), block(256);
    const int vpt = (hidden / 4 + 63) / 64;
#define LNM_CASE(V)                                                                          \
    case V:                                                                                  \
        hipLaunchKernelGGL(ln_modulate_kernel<V>, grid, block, 0, s, x, rows, hidden, split, \
                           shift0, scale0, shift1, scale1, eps, out);                        \
        break;
    switch (vpt) {
        LNM_CASE(1) LNM_CASE(2) LNM_CASE(3) LNM_CASE(4) LNM_CASE(5) LNM_CASE(6) LNM_CASE(7)
        LNM_CASE(8) LNM_CASE(9) LNM_CASE(10) LNM_CASE(11) LNM_CASE(12) LNM_CASE(13)
        LNM_CASE(14) LNM_CASE(15) LNM_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef LNM_CASE
    return hipGetLastError();
}

}  // namespace mmdit
