// Per-head RMSNorm of q and k, axial RoPE, and relayout for attention.
// (Both blocks do this in the epilogue of the projection that makes q, k and
// v when the hidden size is a multiple of 256; this kernel serves other hidden
// sizes and the per-kernel entry.)
//
// Luminal blog, "What the compiler found on its own": RMSNorm is a square, a
// sum, a reciprocal square root and a multiply; RoPE gathers each element's
// partner and multiply-adds it against cosine and sine tables. AMD's SGLang
// Diffusion post ("Architecture Deep Dive") fuses QK normalisation with RoPE
// to save memory round trips; here the fused kernel also writes the layout
// the attention kernel reads, so no separate transpose pass exists:
//   Q, K: [heads, l_pad, D]  (one contiguous D-row per token and head)
//   V^T : [heads, D, l_pad]  (keys along the row; inside each aligned group of
//         16 keys the quads are stored 0, 2, 1, 3, so the 16-byte chunk 2i+j of
//         a group holds keys 4j..4j+3 and 8+4j..8+4j+3 of it: the 8 keys that
//         one lane of the 32x32x16 matrix-core product P V takes, in order)
// Rows in [seq_len, l_pad) are written as zeros so the attention kernel never
// reads past a buffer and padded keys stay finite.
//
// HBM-bound: read 3 * L * H bf16, write the same. A group of D/8 lanes owns
// one (token, head) row of q or k (16-byte loads and stores); the rotated
// pairs (2j, 2j+1) sit inside one lane's 8 elements. V goes through LDS so
// both its read and its transposed write are 16-byte coalesced.
#include "common.h"

namespace mmdit {

template <int D>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    const uint16_t* __restrict__ qkv, int ld, int seq_len, int heads, int split,
    const uint16_t* __restrict__ qn0, const uint16_t* __restrict__ kn0,
    const uint16_t* __restrict__ qn1, const uint16_t* __restrict__ kn1,
    const float* __restrict__ rope, float eps, int l_pad, uint16_t* __restrict__ q_out,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ vt_out) {
    constexpr int CH = D / 8;          // 16-byte chunks per head row
    constexpr int TPP = 256 / CH;      // tokens per pass
    constexpr int TILE = 64;           // tokens per workgroup
    constexpr int LDV = D + 8;         // padded LDS row (elements)
    __shared__ uint16_t vs[TILE * LDV];

    const int h = blockIdx.y;
    const int t0 = blockIdx.x * TILE;
    const int tid = threadIdx.x;
    const int c = tid % CH;
    const int H = heads * D;
    const float inv_d = 1.0f / (float)D;

    // ---- q and k: RMSNorm + RoPE
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        uint16_t* dst = which == 0 ? q_out : k_out;
        for (int p = 0; p < TILE / TPP; ++p) {
            const int t = t0 + p * TPP + tid / CH;
            uint4 res = make_uint4(0u, 0u, 0u, 0u);
            if (t < seq_len) {
                const uint4 raw = *reinterpret_cast<const uint4*>(
                    qkv + (size_t)t * ld + which * H + h * D + c * 8);
                const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw);
                float u[8];
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    u[i] = bf2f(e[i]);
                    ss += u[i] * u[i];
                }
                ss = group_sum<CH>(ss);
                const float rstd = 1.0f / sqrtf(ss * inv_d + eps);
                const uint16_t* g = (t < split) ? (which == 0 ? qn0 : kn0) : (which == 0 ? qn1 : kn1);
                const uint4 graw = *reinterpret_cast<const uint4*>(g + c * 8);
                const uint16_t* ge = reinterpret_cast<const uint16_t*>(&graw);
                const float4* cs = reinterpret_cast<const float4*>(rope + ((size_t)t * (D / 2) + c * 4) * 2);
                const float4 cs0 = cs[0], cs1 = cs[1];
                const float cosv[4] = {cs0.x, cs0.z, cs1.x, cs1.z};
                const float sinv[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = u[2 * j] * rstd * bf2f(ge[2 * j]);
                    const float b = u[2 * j + 1] * rstd * bf2f(ge[2 * j + 1]);
                    w[j] = pack2bf(a * cosv[j] - b * sinv[j], a * sinv[j] + b * cosv[j]);
                }
                res = make_uint4(w[0], w[1], w[2], w[3]);
            }
            if (t < l_pad)
                *reinterpret_cast<uint4*>(dst + ((size_t)h * l_pad + t) * D + c * 8) = res;
        }
    }

    // ---- v: stage the tile in LDS, write it transposed
    for (int idx = tid; idx < TILE * CH; idx += 256) {
        const int r = idx / CH, cc = idx % CH;
        const int t = t0 + r;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (t < seq_len)
            val = *reinterpret_cast<const uint4*>(qkv + (size_t)t * ld + 2 * H + h * D + cc * 8);
        uint32_t* sv = reinterpret_cast<uint32_t*>(vs + r * LDV + cc * 8);
        sv[0] = val.x; sv[1] = val.y; sv[2] = val.z; sv[3] = val.w;
    }
    __syncthreads();
    for (int idx = tid; idx < D * (TILE / 8); idx += 256) {
        const int d = idx / (TILE / 8), tc = idx % (TILE / 8);
        const int tb = t0 + tc * 8;
        if (tb >= l_pad) continue;
        // stored element e of chunk tc is key 16*(tc/2) + 4*(tc%2) + 8*(e/4) + e%4
        const int kb = 16 * (tc >> 1) + 4 * (tc & 1);
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = kb + 8 * (j >> 1) + 2 * (j & 1);
            const uint16_t lo = vs[key * LDV + d];
            const uint16_t hi = vs[(key + 1) * LDV + d];
            w[j] = uint32_t(lo) | (uint32_t(hi) << 16);
        }
        *reinterpret_cast<uint4*>(vt_out + ((size_t)h * D + d) * l_pad + tb) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_qknorm_rope(const uint16_t* qkv, int ld, int seq_len, int heads, int head_dim,
                              int split, const uint16_t* qn0, const uint16_t* kn0,
                              const uint16_t* qn1, const uint16_t* kn1, const float* rope,
                              float eps, int l_pad, uint16_t* q_out, uint16_t* k_out,
                              uint16_t* vt_out, hipStream_t s) {
    dim3 grid(l_pad / 64, heads), block(256);
    if (head_dim == 128)
        hipLaunchKernelGGL(qknorm_rope_kernel<128>, grid, block, 0, s, qkv, ld, seq_len, heads, split,
                           qn0, kn0, qn1, kn1, rope, eps, l_pad, q_out, k_out, vt_out);
    else if (head_dim == 64)
        hipLaunchKernelGGL(qknorm_rope_kernel<64>, grid, block, 0, s, qkv, ld, seq_len, heads, split,
                           qn0, kn0, qn1, kn1, rope, eps, l_pad, q_out, k_out, vt_out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mmdit
