// fp8 attention: the attention products on gfx950's fp8 matrix cores.
//
// SGLang-AMD blog, "Architecture Deep Dive": fp8 quantisation on the CDNA
// stack; Luminal blog, "What the compiler found on its own": attention is two
// matrix products around a scaled softmax. The fp8 form computed here:
// * q and k as OCP e4m3 codes at one power-of-two scale per tensor, 2^eq and
//   2^ek. After QK-RMSNorm (and RoPE, a rotation) every element satisfies
//   |x| <= sqrt(D) * max|g| with g the norm scale, so the scale is the
//   smallest power of two at or above sqrt(D) * max|g| / 448: no code can
//   overflow, and a power of two makes the scaling exact;
// * v^T as e4m3 codes with one fp32 scale per channel (head dimension),
//   max over the tokens of |v| / 448, applied once to each output element;
// * logits in log2 units t = (q8 . k8) 2^(eq+ek) log2(e) / sqrt(D); the
//   exponentials p = 2^(t - M + 8) against an integer reference M at or
//   above the row maximum seen so far, so p lies in [0, 256]; the second
//   product takes e4m3(p) and the row sum the fp32 p. M moves (to the ceiling
//   of the new maximum) whenever a tile's maximum exceeds it; because M is an
//   integer, the codes of earlier tiles differ from codes against the final M
//   by exact powers of two (e4m3 rounding commutes with them in its normal
//   range), so the tiled result equals the definition against the row's true
//   maximum up to fp32 rounding.
//
// gfx950 design: the bf16 kernel's structure (8 wavefronts x 32 query rows,
// 64-key tiles double-buffered in LDS with 16-byte direct-to-LDS loads, S^T =
// K Q^T so each lane owns one query row's 32 scores of a tile) with
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): lane l of an operand
// holds row l%32 and the 32 consecutive k-bytes 32(l/32) .. +31 (checked on
// the GPU against a CPU product). QK^T: D/64 products per 32-key half; PV: one
// product per 32 output channels. The probabilities are converted in
// registers into exactly the second operand's layout: slot j of lane (r, g)
// is the lane's own score j (half j/16, element j%16), i.e. key
// 32(j/16) + 8((j%16)/4) + 4g + j%4; v^T is stored in HBM with the keys of
// each 64-key tile in that slot order, so one lane's operand is 32
// contiguous bytes.
#include "common.h"

namespace mmdit {

namespace {
typedef __attribute__((address_space(3))) void lds_void8;
MMDIT_DEV void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// 16-byte direct global -> LDS load (lane i writes lds_base + 16 i)
MMDIT_DEV void g2l16(const void* gsrc, lds_void8* lds_base) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(gsrc) : "memory", "m0");
}
MMDIT_DEV i32x8_t lds32(const char* p0, const char* p1) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p0);
    const uint4 hi = *reinterpret_cast<const uint4*>(p1);
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// max|g| over one or two norm-scale vectors of n <= 256 entries, reduced over
// a 256-thread workgroup (every thread gets the result)
MMDIT_DEV float block_absmax_bf16(const uint16_t* g0, const uint16_t* g1, int n, float* red) {
    const int t = threadIdx.x;
    float m = 0.f;
    if (t < n) {
        m = fabsf(bf2f(g0[t]));
        if (g1) m = fmaxf(m, fabsf(bf2f(g1[t])));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __syncthreads();
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
}  // namespace

template <int D>
struct Attn8Tile {
    static constexpr int KV = 64;
    static constexpr int RB = D;                 // bytes per K row
    static constexpr int CPR = D / 16;           // 16-byte chunks per K row
    static constexpr int K_BYTES = KV * RB;
    static constexpr int V_BYTES = D * KV;       // D rows of 64 bytes
    static constexpr int K_LOADS = K_BYTES / 1024;   // 1 KB wavefront loads per tile
    static constexpr int V_LOADS = V_BYTES / 1024;
    static constexpr int LPW = (K_LOADS + V_LOADS) / 8;   // loads per wavefront per tile
    static constexpr int K_ROWS_PER_LOAD = 1024 / RB;
    // K row r keeps chunk c at c ^ ksw(r): the 16 rows one 16-lane read group
    // touches land on 16 distinct 16-byte bank groups
    static MMDIT_DEV int ksw(int r) { return (r / (256 / RB)) & (CPR - 1); }
    static MMDIT_DEV int vsw(int d) { return (d >> 2) & 3; }
};

template <int D>
__global__ __launch_bounds__(512, 1) void attention_fp8_kernel(const uint8_t* __restrict__ q,
                                                               const uint8_t* __restrict__ k,
                                                               const uint8_t* __restrict__ vt,
                                                               const float* __restrict__ sv,
                                                               const int* __restrict__ exps,
                                                               int seq_len, int l_pad, int heads,
                                                               uint16_t* __restrict__ out, int ldo,
                                                               float c_log2) {
    using T = Attn8Tile<D>;
    __shared__ __attribute__((aligned(1024))) char sK0[T::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char sV0[T::V_BYTES];
    __shared__ __attribute__((aligned(1024))) char sK1[T::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char sV1[T::V_BYTES];

    const int nq = (seq_len + 255) / 256;
    const int total = nq * heads;
    int bid = blockIdx.x;
    if (total % 8 == 0) bid = (bid % 8) * (total / 8) + bid / 8;   // a head's K/V through one XCD's L2
    const int h = bid / nq, qt = bid % nq;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, r32 = lane & 31;
    const int qrow = qt * 256 + wave * 32 + r32;
    const float cl = c_log2 * ldexpf(1.0f, exps[0] + exps[1]);

    // Q^T fragments: lane (r32, g) holds bytes kk*64 + 32g .. +31 of its row
    const int qld = qrow < l_pad ? qrow : l_pad - 1;
    const uint8_t* qp = q + ((size_t)h * l_pad + qld) * D + g * 32;
    i32x8_t qf[D / 64];
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) qf[kk] = lds32((const char*)(qp + kk * 64), (const char*)(qp + kk * 64 + 16));
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) asm volatile("" ::"v"(qf[kk].lo), "v"(qf[kk].hi));   // 128-bit halves

    // load descriptors (wave-uniform choice of K or V load)
    const char* kbase = reinterpret_cast<const char*>(k + (size_t)h * l_pad * D);
    const char* vbase = reinterpret_cast<const char*>(vt + (size_t)h * D * l_pad);
    uint32_t src[T::LPW];
    int dst[T::LPW];
    bool isk[T::LPW];
#pragma unroll
    for (int j = 0; j < T::LPW; ++j) {
        const int li = wave * T::LPW + j;
        isk[j] = li < T::K_LOADS;
        if (isk[j]) {
            const int r = li * T::K_ROWS_PER_LOAD + lane / T::CPR;
            const int c = (lane % T::CPR) ^ T::ksw(r);
            src[j] = (uint32_t)(r * T::RB + c * 16);
            dst[j] = li * 1024;
        } else {
            const int vl = li - T::K_LOADS;
            const int d = vl * 16 + lane / 4;
            const int c = (lane % 4) ^ T::vsw(d);
            src[j] = (uint32_t)d * (uint32_t)l_pad + (uint32_t)(c * 16);
            dst[j] = vl * 1024;
        }
    }
    auto issue = [&](int t, char* sK, char* sV) {
#pragma unroll
        for (int j = 0; j < T::LPW; ++j) {
            if (isk[j])
                g2l16(kbase + (src[j] + (uint32_t)t * T::KV * T::RB), (lds_void8*)(sK + dst[j]));
            else
                g2l16(vbase + (src[j] + (uint32_t)t * T::KV), (lds_void8*)(sV + dst[j]));
        }
    };

    // fragment offsets: K rows st*32 + r32, chunks 4kk + 2g + {0,1};
    // V^T rows dt*32 + r32, chunks 2g + {0,1}
    int k_off[2][D / 64][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int row = st * 32 + r32;
                const int c = 4 * kk + 2 * g + hh;
                k_off[st][kk][hh] = row * T::RB + ((c ^ T::ksw(row)) * 16);
            }
    int v_off[D / 32][2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int d = dt * 32 + r32;
            v_off[dt][hh] = d * 64 + (((2 * g + hh) ^ T::vsw(d)) * 16);
        }

    f32x16_t o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // m_run: integer reference (log2 units)
    const int nkv = (seq_len + T::KV - 1) / T::KV;

    auto compute = [&](int t, const char* sK, const char* sV) {
        f32x16_t s[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk) {
                const i32x8_t kf = lds32(sK + k_off[st][kk][0], sK + k_off[st][kk][1]);
                s[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[kk], s[st], 0, 0, 0, 127, 0, 127);
            }
        }
        // element i of s[st]: key t*64 + st*32 + 8*(i/4) + 4g + i%4
        const int kv0 = t * T::KV;
        if (kv0 + T::KV > seq_len) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kv0 + st * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key >= seq_len) s[st][i] = -INFINITY;
                }
        }
        float tmax = s[0][0];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[st][i]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float cand = tmax * cl;
        const bool move = cand > m_run;
        const float m_new = move ? ceilf(cand) : m_run;
        const bool any_move = __ballot(move) != 0ull;   // wave-uniform
        float alpha = 1.0f;
        if (any_move) alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        const float sub = m_new - 8.0f;
        float psum = 0.f;
        i32x8_t pf;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int st = w >> 2, i0 = (w & 3) * 4;
            float p[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                p[u] = __builtin_amdgcn_exp2f(s[st][i0 + u] * cl - sub);
                psum += p[u];
            }
            uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0u, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], pk, true);
            pf[w] = (int)pk;
        }
        l_run = l_run * alpha + psum;
        if (any_move) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const i32x8_t vf = lds32(sV + v_off[dt][0], sV + v_off[dt][1]);
            o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[dt], 0, 0, 0, 127, 0, 127);
        }
    };

    issue(0, sK0, sV0);
    wait_vm0();
    __syncthreads();
    for (int t = 0; t < nkv; t += 2) {
        if (t + 1 < nkv) issue(t + 1, sK1, sV1);
        compute(t, sK0, sV0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm0();
        __syncthreads();
        if (t + 1 >= nkv) break;
        if (t + 2 < nkv) issue(t + 2, sK0, sV0);
        compute(t + 1, sK1, sV1);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm0();
        __syncthreads();
    }

    // o[dt] element i is O[qrow][dt*32 + 8*(i/4) + 4g + i%4] / (channel scale)
    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = 1.0f / l_tot;
    if (qrow < seq_len) {
        uint16_t* op = out + (size_t)qrow * ldo + h * D + 4 * g;
        const float* svp = sv + h * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const float4 c = *reinterpret_cast<const float4*>(svp + dt * 32 + 8 * i4);
                const uint2 w = make_uint2(pack2h(o[dt][4 * i4] * inv * c.x, o[dt][4 * i4 + 1] * inv * c.y),
                                           pack2h(o[dt][4 * i4 + 2] * inv * c.z, o[dt][4 * i4 + 3] * inv * c.w));
                *reinterpret_cast<uint2*>(op + dt * 32 + 8 * i4) = w;
            }
    }
}

// q and k (bf16 [heads, l_pad, D] each) to e4m3 codes at their power-of-two
// scales. Every workgroup derives both exponents from the norm scales (at
// most 4 x D reads); workgroup 0 also stores them for the attention kernel.
__global__ __launch_bounds__(256) void quantize_qk_fp8_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k, int64_t n16,
                                                             const uint16_t* gq0, const uint16_t* gq1,
                                                             const uint16_t* gk0, const uint16_t* gk1,
                                                             int head_dim, float bound_factor,
                                                             uint8_t* __restrict__ q8, uint8_t* __restrict__ k8,
                                                             int* __restrict__ exps) {
    __shared__ float red[4];
    const float gq = block_absmax_bf16(gq0, gq1, head_dim, red);
    const float gk = block_absmax_bf16(gk0, gk1, head_dim, red);
    const int eq = ceil_log2_exp(bound_factor * gq), ek = ceil_log2_exp(bound_factor * gk);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        exps[0] = eq;
        exps[1] = ek;
    }
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n16; i += stride) {
        const bool isq = i < n16;
        const int64_t j = isq ? i : i - n16;
        const uint4* src = reinterpret_cast<const uint4*>(isq ? q : k) + 2 * j;
        const float sc = ldexpf(1.0f, -(isq ? eq : ek));
        const uint4 a = src[0], b = src[1];
        const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t pk[4];
        // |x| 2^-e <= 448 by the RMSNorm bound; the clamp only keeps a value
        // that its own bf16 rounding pushed just past 448 (below 464, where
        // rounding to nearest gives 448 anyway) out of the conversion's
        // overflow range
        auto c448 = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t w0 = wv[2 * u], w1 = wv[2 * u + 1];
            uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(c448(bf2f(w0 & 0xffffu) * sc), c448(bf2f(w0 >> 16) * sc),
                                                         0u, false);
            pk[u] = __builtin_amdgcn_cvt_pk_fp8_f32(c448(bf2f(w1 & 0xffffu) * sc), c448(bf2f(w1 >> 16) * sc), p,
                                                    true);
        }
        reinterpret_cast<uint4*>(isq ? q8 : k8)[j] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
}

// v^T (bf16 [rows = heads*D, l_pad], the bf16 attention's quad-swapped key
// order) to e4m3 codes in the fp8 slot order with one scale per row
// (channel): scale = max|v| / 448, code = e4m3(v / scale), both in fp32.
// One workgroup per row: the maximum, then the codes (the second read hits L2).
__global__ __launch_bounds__(256) void quantize_vt_fp8_kernel(const uint16_t* __restrict__ vt, int l_pad,
                                                             uint8_t* __restrict__ vt8, float* __restrict__ sv) {
    __shared__ float red[4];
    const int row = blockIdx.x;
    const uint2* src = reinterpret_cast<const uint2*>(vt + (size_t)row * l_pad);   // 4 keys per uint2
    const int nquad = l_pad / 4;
    float amax = 0.f;
    for (int i = threadIdx.x; i < nquad; i += 256) {
        const uint2 w = src[i];
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf2f(w.x & 0xffffu)), fabsf(bf2f(w.x >> 16))),
                                 fmaxf(fabsf(bf2f(w.y & 0xffffu)), fabsf(bf2f(w.y >> 16)))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 448.0f;
    if (threadIdx.x == 0) sv[row] = s;
    uint32_t* dstw = reinterpret_cast<uint32_t*>(vt8 + (size_t)row * l_pad);
    // output dword w of a tile holds slots 4w .. 4w+3 = keys 32 st + 8 a + 4 g + {0..3},
    // w = 8 g + 4 st + a; in the bf16 order the key quad kq (0..3 within its
    // 16 keys) sits at quad position kq with 1 and 2 exchanged
    for (int w = threadIdx.x; w < nquad; w += 256) {
        const int tile = w >> 4, wt = w & 15;
        const int gg = wt >> 3, st = (wt >> 2) & 1, a = wt & 3;
        const int key = tile * 64 + st * 32 + a * 8 + gg * 4;
        const int kq = (key >> 2) & 3;
        const int pos = (key & ~15) | ((((kq & 1) << 1) | (kq >> 1)) << 2);
        const uint2 v = src[pos >> 2];
        uint32_t pk = 0u;
        if (s > 0.f) {
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(bf2f(v.x & 0xffffu) / s, bf2f(v.x >> 16) / s, 0u, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(bf2f(v.y & 0xffffu) / s, bf2f(v.y >> 16) / s, pk, true);
        }
        dstw[w] = pk;
    }
}

hipError_t launch_quantize_attention_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int heads,
                                         int head_dim, int l_pad, const uint16_t* gq0, const uint16_t* gq1,
                                         const uint16_t* gk0, const uint16_t* gk1, uint8_t* q8, uint8_t* k8,
                                         uint8_t* vt8, float* sv, int* exps, hipStream_t s) {
    if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
    if (l_pad <= 0 || l_pad % 64 != 0 || heads <= 0 || !gq0 || !gk0) return hipErrorInvalidValue;
    const int64_t n16 = (int64_t)heads * l_pad * head_dim / 16;
    const float bound_factor = (float)(sqrt((double)head_dim) / 448.0);
    const int64_t want = (2 * n16 + 255) / 256;
    dim3 grid((unsigned)(want < 2048 ? want : 2048)), block(256);
    hipLaunchKernelGGL(quantize_qk_fp8_kernel, grid, block, 0, s, q, k, n16, gq0, gq1, gk0, gk1, head_dim,
                       bound_factor, q8, k8, exps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quantize_vt_fp8_kernel, dim3(heads * head_dim), block, 0, s, vt, l_pad, vt8, sv);
    return hipGetLastError();
}

hipError_t launch_quantize_vt_fp8(const uint16_t* vt, int heads, int head_dim, int l_pad, uint8_t* vt8, float* sv,
                                  hipStream_t s) {
    if ((head_dim != 64 && head_dim != 128) || l_pad <= 0 || l_pad % 64 != 0 || heads <= 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_vt_fp8_kernel, dim3(heads * head_dim), dim3(256), 0, s, vt, l_pad, vt8, sv);
    return hipGetLastError();
}

hipError_t launch_attention_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, const float* sv,
                                const int* exps, int heads, int seq_len, int head_dim, int l_pad, uint16_t* out,
                                int ldo, hipStream_t s) {
    if (seq_len <= 0) return hipSuccess;
    if (l_pad >= (1 << 24) || l_pad % 64 != 0 || l_pad < seq_len) return hipErrorInvalidValue;
    dim3 grid(((seq_len + 255) / 256) * heads), block(512);
    const float c_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
    if (head_dim == 128)
        hipLaunchKernelGGL(attention_fp8_kernel<128>, grid, block, 0, s, q8, k8, vt8, sv, exps, seq_len, l_pad, heads,
                           out, ldo, c_log2);
    else if (head_dim == 64)
        hipLaunchKernelGGL(attention_fp8_kernel<64>, grid, block, 0, s, q8, k8, vt8, sv, exps, seq_len, l_pad, heads,
                           out, ldo, c_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mmdit
