// LayerNorm + adaLN modulate: fp32 residual rows -> fp16 GEMM operand.
//
// Luminal blog, "What the compiler found on its own": LayerNorm is a mean, a
// subtraction, a square-sum and a reciprocal square root; the adaLN
// modulation after it is a scale and a shift. Here: out = LN(x)(1+scale)+shift
// with a biased variance and no affine.
//
// The output is the activation operand of the next projection, stored as
// fp16 (10-bit significand; LayerNorm outputs are O(10), far inside fp16's
// range; a value beyond +-65504 is stored as +-inf, the IEEE conversion).
// HBM-bound: each row is read once (4 B/elem), written once (2 B/elem).
// A row is held in registers by one, two or four wavefronts (up to four float4
// per lane), so the two-pass mean/variance costs no second HBM read. Wide rows
// (FLUX's 3072) take a whole workgroup per row. 128-bit loads, 64-bit stores,
// DPP reductions within the wavefront.
#include "common.h"

namespace mmdit {

// W wavefronts share one row (W = 1, 2 or 4, so a 256-thread workgroup holds
// 4/W rows at a time); lane t of wave w holds float4 columns (i*W + w)*64 + t.
// The two sums are reduced within each wavefront (DPP, no LDS round trip),
// then over the row's W partials in LDS in a fixed order, so the result does
// not depend on timing. Each workgroup streams rows (a fixed grid, rows
// strided by the grid): the next rows' loads are issued before the current
// rows are reduced, so the HBM stream does not drain between rows; the
// shift/scale vectors of both row groups (text / image) are loaded once.
// FP8: the row goes out as OCP e4m3 codes with one fp32 scale instead of
// fp16 (the projection's fp8 operand): the fp16 rounding of each output is
// kept, then scale = max|h| / 448 and code = e4m3(h / scale), both divisions
// in fp32 and the conversion round-to-nearest-even, exactly as the separate
// per-row quantiser does on the fp16 row (bit-identical codes and scales).
template <int VPT, int W, bool FP8>
__global__ __launch_bounds__(256) void ln_modulate_kernel(
    const float* __restrict__ x, int rows, int hidden, int split,
    const float* __restrict__ shift0, const float* __restrict__ scale0,
    const float* __restrict__ shift1, const float* __restrict__ scale1, float eps,
    uint16_t* __restrict__ out, uint8_t* __restrict__ codes, float* __restrict__ qscale) {
    __shared__ float red[3][4];
    constexpr int RPB = 4 / W;                     // rows per workgroup per iteration
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = wave % W;                      // this wave's part of the row
    const int n4 = hidden >> 2;
    const int step = gridDim.x * RPB;
    const float inv_h = 1.0f / (float)hidden;
    int col[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) col[i] = (i * W + sub) * 64 + lane;
    // both groups' shift and scale, once (columns past the row clamp to 0)
    float4 sh[2][VPT], sc[2][VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = col[i] < n4 ? col[i] : 0;
        sh[0][i] = reinterpret_cast<const float4*>(shift0)[c];
        sc[0][i] = reinterpret_cast<const float4*>(scale0)[c];
        sh[1][i] = reinterpret_cast<const float4*>(shift1)[c];
        sc[1][i] = reinterpret_cast<const float4*>(scale1)[c];
    }
    auto load = [&](int row, float4 (&v)[VPT]) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)(row < rows ? row : rows - 1) * hidden);
#pragma unroll
        for (int i = 0; i < VPT; ++i) v[i] = xr[col[i] < n4 ? col[i] : 0];
    };
    int row = blockIdx.x * RPB + wave / W;
    float4 v[VPT], vn[VPT];
    load(row, v);
    // the workgroup iterates while its first row is valid (uniform, so every
    // wavefront meets the same barriers); rows past the end are not stored
    for (int first = blockIdx.x * RPB; first < rows; first += step, row += step) {
        load(row + step, vn);
        const bool valid = row < rows;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            if (col[i] >= n4) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        }
        s = wave_sum(s);
        if (W > 1) {
            if (lane == 0) red[0][wave] = s;
            __syncthreads();
            const int w0 = wave - sub;
            s = red[0][w0];
#pragma unroll
            for (int w = 1; w < W; ++w) s += red[0][w0 + w];
        }
        const float mean = s * inv_h;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            if (col[i] < n4) {
                const float a = v[i].x - mean, b = v[i].y - mean, cc = v[i].z - mean, d = v[i].w - mean;
                q += (a * a + b * b) + (cc * cc + d * d);
            }
        }
        q = wave_sum(q);
        if (W > 1) {
            if (lane == 0) red[1][wave] = q;
            __syncthreads();
            const int w0 = wave - sub;
            q = red[1][w0];
#pragma unroll
            for (int w = 1; w < W; ++w) q += red[1][w0 + w];
        }
        const float rstd = 1.0f / sqrtf(q * inv_h + eps);
        const int grp = row < split ? 0 : 1;
        uint2* orow = reinterpret_cast<uint2*>(out + (size_t)(valid ? row : 0) * hidden);
        uint2 hv[VPT];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = col[i];
            hv[i] = make_uint2(0u, 0u);
            if (c < n4) {
                const float4 a = grp ? sh[1][i] : sh[0][i], b = grp ? sc[1][i] : sc[0][i];
                const float y0 = (v[i].x - mean) * rstd * (1.0f + b.x) + a.x;
                const float y1 = (v[i].y - mean) * rstd * (1.0f + b.y) + a.y;
                const float y2 = (v[i].z - mean) * rstd * (1.0f + b.z) + a.z;
                const float y3 = (v[i].w - mean) * rstd * (1.0f + b.w) + a.w;
                hv[i] = make_uint2(pack2h(y0, y1), pack2h(y2, y3));
                if (!FP8) {
                    if (valid) orow[c] = hv[i];
                } else {
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(h2f(hv[i].x & 0xffffu)), fabsf(h2f(hv[i].x >> 16))),
                                             fmaxf(fabsf(h2f(hv[i].y & 0xffffu)), fabsf(h2f(hv[i].y >> 16)))));
                }
            }
        }
        if constexpr (FP8) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            if (W > 1) {
                if (lane == 0) red[2][wave] = amax;
                __syncthreads();
                const int w0 = wave - sub;
#pragma unroll
                for (int w = 0; w < W; ++w) amax = fmaxf(amax, red[2][w0 + w]);
            }
            const float qs = amax / 448.0f;
            uint32_t* crow = reinterpret_cast<uint32_t*>(codes + (size_t)(valid ? row : 0) * hidden);
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int c = col[i];
                if (c < n4 && valid) {
                    uint32_t packed = 0u;
                    if (qs > 0.f) {
                        packed = __builtin_amdgcn_cvt_pk_fp8_f32(h2f(hv[i].x & 0xffffu) / qs,
                                                                 h2f(hv[i].x >> 16) / qs, 0u, false);
                        packed = __builtin_amdgcn_cvt_pk_fp8_f32(h2f(hv[i].y & 0xffffu) / qs,
                                                                 h2f(hv[i].y >> 16) / qs, packed, true);
                    }
                    crow[c] = packed;
                }
            }
            if (valid && sub == 0 && lane == 0) qscale[row] = qs;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) v[i] = vn[i];
    }
}

hipError_t launch_ln_modulate(const float* x, int rows, int hidden, int split,
                              const float* shift0, const float* scale0,
                              const float* shift1, const float* scale1, float eps,
                              uint16_t* out, hipStream_t s, uint8_t* codes, float* qscale) {
    if (rows <= 0) return hipSuccess;
    if (hidden < 64 || hidden % 64 != 0 || hidden > 4096) return hipErrorInvalidValue;
    const int n4 = hidden / 4;
    const int w = n4 >= 512 ? 4 : n4 >= 256 ? 2 : 1;   // VPT = 1..4 in every case
    const int vpt = (n4 + 64 * w - 1) / (64 * w);
    // a fixed grid of at most 1024 workgroups, each streaming an equal number
    // (+-1) of row groups
    const int row_blocks = (rows + 4 / w - 1) / (4 / w);
    const int iters = (row_blocks + 1023) / 1024;
    dim3 grid((row_blocks + iters - 1) / iters), block(256);
#define LNM_CASE(V, WW)                                                                        \
    if (vpt == V && w == WW) {                                                                 \
        if (codes)                                                                             \
            hipLaunchKernelGGL((ln_modulate_kernel<V, WW, true>), grid, block, 0, s, x, rows, hidden, split, \
                               shift0, scale0, shift1, scale1, eps, out, codes, qscale);       \
        else                                                                                   \
            hipLaunchKernelGGL((ln_modulate_kernel<V, WW, false>), grid, block, 0, s, x, rows, hidden, split, \
                               shift0, scale0, shift1, scale1, eps, out, codes, qscale);       \
        return hipGetLastError();                                                              \
    }
    LNM_CASE(1, 1) LNM_CASE(2, 1) LNM_CASE(3, 1) LNM_CASE(4, 1)
    LNM_CASE(2, 2) LNM_CASE(3, 2) LNM_CASE(4, 2)
    LNM_CASE(2, 4) LNM_CASE(3, 4) LNM_CASE(4, 4)
#undef LNM_CASE
    return hipErrorInvalidValue;
}

}  // namespace mmdit
