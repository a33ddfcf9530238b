// Small kernels around the block: the vector-matrix products of the
// modulation and embedder layers, the sinusoidal timestep embedding, the
// Euler update, the RoPE table and a plain copy.
#include "common.h"

namespace mmdit {

// ---------------------------------------------------------------------------
// out_g[r] (+)= sum_k W_g[r,k] act(x[k]) + b_g[r], r < n, for one or two
// weight sets g that share the input x (the text and image stream
// modulations of a double block share the conditioning vector).
//
// Pure weight streaming (HBM-bound: 2 B per weight in bf16/fp16, 1 B in
// int8). Lane l owns the columns l*E + i*64*E (E = 8 16-bit or 16 int8
// weights = one 16-byte load, i < NL) of every row and keeps act(x) of those
// columns in registers. A fixed grid of wavefronts streams the rows in
// groups of GEMV_RPW: each wavefront issues the loads of its next group
// before it reduces the current one, so the weight stream never drains
// (226 MB of cold modulation weights: 5.6 TB/s against 3.3 TB/s for one
// short-lived wavefront per group, measured). Every weight is read once per
// call, so the loads are nontemporal: they do not allocate in the caches,
// which after a large write are full of dirty lines (226 MB after a 1 GiB
// fill: 46 us against 91 us with ordinary loads, bit-identical).
// ---------------------------------------------------------------------------
constexpr int GEMV_RPW = 2;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int GEMV_MAX_BLOCKS = 512;

template <int WT, int NL>
__global__ __launch_bounds__(256) void gemv_kernel(const float* __restrict__ x, int k, int n,
                                                   int silu_input, int accumulate, const GemvSets sets) {
    constexpr bool INT8 = WT == MMDIT_INT8;
    constexpr bool FP8 = WT == MMDIT_FP8;
    constexpr bool BYTE = INT8 || FP8;  // one byte per weight, a scale per row
    constexpr int E = BYTE ? 16 : 8;
    constexpr int ES = BYTE ? 1 : 2;   // bytes per weight
    const int lane = threadIdx.x & 63;
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nw = gridDim.x * 4;
    const int rows = sets.count * n;
    const int groups = (rows + GEMV_RPW - 1) / GEMV_RPW;
    if (wv >= groups) return;
    float xs[NL][E];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int c = lane * E + i * 64 * E;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < k) v = *reinterpret_cast<const float4*>(x + c + 4 * q);
            if (silu_input) { v.x = silu(v.x); v.y = silu(v.y); v.z = silu(v.z); v.w = silu(v.w); }
            xs[i][4 * q] = v.x; xs[i][4 * q + 1] = v.y; xs[i][4 * q + 2] = v.z; xs[i][4 * q + 3] = v.w;
        }
    }
    // Loads from clamped, always valid addresses (a row past the end re-reads
    // the last row and is not stored; columns past k meet act(x) = 0), so the
    // loads are straight-line code. The row's bias, scale and (accumulating)
    // previous output are loaded with its weights: a load issued later, in the
    // reduction, would make the wait before it drain the next group's weight
    // loads too (the counter of outstanding loads is in issue order).
    struct RowExtra { float bias, scale, prev; };
    auto load = [&](int g, uint4 (&raw)[GEMV_RPW][NL], RowExtra (&ex)[GEMV_RPW]) {
#pragma unroll
        for (int rr = 0; rr < GEMV_RPW; ++rr) {
            int row = g * GEMV_RPW + rr;
            row = row < rows ? row : rows - 1;
            const int s = row < n ? 0 : 1;
            const int r = row - s * n;
            const char* wr = static_cast<const char*>(sets.s[s].w) + (size_t)r * k * ES;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                int c = lane * E + i * 64 * E;
                c = c < k ? c : 0;
                const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wr + c * ES));
                raw[rr][i] = make_uint4(t.x, t.y, t.z, t.w);
            }
            ex[rr].bias = bf2f(sets.s[s].bias[r]);
            ex[rr].scale = BYTE ? sets.s[s].scale[r] : 1.0f;
            ex[rr].prev = accumulate ? sets.s[s].out[r] : 0.0f;
        }
    };
    auto reduce = [&](int g, const uint4 (&raw)[GEMV_RPW][NL], const RowExtra (&ex)[GEMV_RPW]) {
#pragma unroll
        for (int rr = 0; rr < GEMV_RPW; ++rr) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                if (INT8) {
                    const int8_t* e = reinterpret_cast<const int8_t*>(&raw[rr][i]);
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc += (float)e[j] * xs[i][j];
                } else if (FP8) {
                    // e4m3 codes -> fp32 (exact), two per conversion
                    const uint32_t w[4] = {raw[rr][i].x, raw[rr][i].y, raw[rr][i].z, raw[rr][i].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);
                        acc += lo[0] * xs[i][4 * j] + lo[1] * xs[i][4 * j + 1];
                        acc += hi[0] * xs[i][4 * j + 2] + hi[1] * xs[i][4 * j + 3];
                    }
                } else if (WT == MMDIT_F16) {
                    // fp16 -> fp32 is exact; converted by the hardware (a bit
                    // rescale with the sign patched in took ~4 VALU operations
                    // per weight: 21.0 -> 19.6 us per 113 MB, bit-identical)
                    const _Float16* e = reinterpret_cast<const _Float16*>(&raw[rr][i]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc += static_cast<float>(e[j]) * xs[i][j];
                } else {
                    const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw[rr][i]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc += bf2f(e[j]) * xs[i][j];
                }
            }
            acc = wave_sum(acc);
            const int row = g * GEMV_RPW + rr;
            if (lane == 0 && row < rows) {
                const int s = row < n ? 0 : 1, r = row - s * n;
                const float y = (BYTE ? acc * ex[rr].scale : acc) + ex[rr].bias;
                sets.s[s].out[r] = accumulate ? ex[rr].prev + y : y;
            }
        }
    };
    // two register buffers in turn: the loads of group g + nw are in flight
    // while group g is reduced
    // (A wave's last prefetch re-reads its current group when no next group
    // is left: the loads stay unconditional, the re-read is never reduced.)
    uint4 ra[GEMV_RPW][NL], rb[GEMV_RPW][NL];
    RowExtra ea[GEMV_RPW], eb[GEMV_RPW];
    load(wv, ra, ea);
    for (int g = wv; g < groups; g += 2 * nw) {
        load(g + nw < groups ? g + nw : g, rb, eb);
        reduce(g, ra, ea);
        if (g + nw >= groups) break;
        load(g + 2 * nw < groups ? g + 2 * nw : g + nw, ra, ea);
        reduce(g + nw, rb, eb);
    }
}


hipError_t launch_gemv(const float* x, int k, int n, int wtype, int silu_input, int accumulate,
                       const GemvSets& sets, hipStream_t s) {
    if (n <= 0 || sets.count < 1) return hipSuccess;
    const int E = (wtype == MMDIT_INT8 || wtype == MMDIT_FP8) ? 16 : 8;
    const int nl = (k + 64 * E - 1) / (64 * E);
    const int groups = (sets.count * n + GEMV_RPW - 1) / GEMV_RPW;
    int blocks = (groups + 3) / 4;
    if (blocks > GEMV_MAX_BLOCKS) blocks = GEMV_MAX_BLOCKS;
    const dim3 grid(blocks), block(256);
#define GEMV_CASE(T, L)                                                                                  \
    if (wtype == T && nl == L) {                                                                         \
        hipLaunchKernelGGL((gemv_kernel<T, L>), grid, block, 0, s, x, k, n, silu_input, accumulate, sets); \
        return hipGetLastError();                                                                        \
    }
    GEMV_CASE(MMDIT_BF16, 1) GEMV_CASE(MMDIT_BF16, 2) GEMV_CASE(MMDIT_BF16, 3) GEMV_CASE(MMDIT_BF16, 4)
    GEMV_CASE(MMDIT_BF16, 5) GEMV_CASE(MMDIT_BF16, 6) GEMV_CASE(MMDIT_BF16, 7) GEMV_CASE(MMDIT_BF16, 8)
    GEMV_CASE(MMDIT_F16, 1) GEMV_CASE(MMDIT_F16, 2) GEMV_CASE(MMDIT_F16, 3) GEMV_CASE(MMDIT_F16, 4)
    GEMV_CASE(MMDIT_F16, 5) GEMV_CASE(MMDIT_F16, 6) GEMV_CASE(MMDIT_F16, 7) GEMV_CASE(MMDIT_F16, 8)
    GEMV_CASE(MMDIT_INT8, 1) GEMV_CASE(MMDIT_INT8, 2) GEMV_CASE(MMDIT_INT8, 3) GEMV_CASE(MMDIT_INT8, 4)
    GEMV_CASE(MMDIT_FP8, 1) GEMV_CASE(MMDIT_FP8, 2) GEMV_CASE(MMDIT_FP8, 3) GEMV_CASE(MMDIT_FP8, 4)
#undef GEMV_CASE
    return hipErrorInvalidValue;
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
// Per-row fp8 quantisation (OCP e4m3, largest finite 448): scale = max|x| /
// 448, code = e4m3(x / scale), both divisions correctly rounded fp32, the
// conversion round-to-nearest-even (v_cvt_pk_fp8_f32). One 256-thread
// workgroup per row; 8 values per thread and pass (16-byte loads, 8-byte
// stores); the row is read twice (the second pass from L2).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_fp8_rows_kernel(const uint16_t* __restrict__ x, int x_bf16,
                                                                int cols, int ldx, uint8_t* __restrict__ codes,
                                                                int ldc, float* __restrict__ scales) {
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * ldx);
    const int n8 = cols >> 3;
    auto val = [&](uint32_t bits) -> float { return x_bf16 ? bf2f((uint16_t)bits) : h2f((uint16_t)bits); };
    float m = 0.f;
    for (int c = tid; c < n8; c += 256) {
        const uint4 v = xr[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(val(w[i] & 0xffffu)), fabsf(val(w[i] >> 16))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = m / 448.0f;
    uint2* cr = reinterpret_cast<uint2*>(codes + (size_t)row * ldc);
    for (int c = tid; c < n8; c += 256) {
        const uint4 v = xr[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
        if (sc > 0.f) {
            float q[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                q[2 * i] = val(w[i] & 0xffffu) / sc;
                q[2 * i + 1] = val(w[i] >> 16) / sc;
            }
            // codes 0-3 into word 0 (low half, then high half), 4-7 into word 1
            packed[0] = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0u, false);
            packed[0] = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], packed[0], true);
            packed[1] = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0u, false);
            packed[1] = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], packed[1], true);
        }
        cr[c] = make_uint2(packed[0], packed[1]);
    }
    if (tid == 0) scales[row] = sc;
}

hipError_t launch_quantize_fp8_rows(const uint16_t* x, bool x_bf16, int rows, int cols, int ldx,
                                    uint8_t* codes, int ldc, float* scales, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3(rows), dim3(256), 0, s, x, x_bf16 ? 1 : 0, cols, ldx, codes,
                       ldc, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// out fp16 [rows, n] = SiLU(x fp32 [rows, n]): the activation operand of the
// modulation linears when they run as one GEMM over many conditioning vectors
// ---------------------------------------------------------------------------
__global__ void silu_to_f16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        y[i] = f2h(silu(x[i]));
}

hipError_t launch_silu_to_f16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(silu_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, n);
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
